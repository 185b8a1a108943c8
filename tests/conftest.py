import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


# Figures a test reports (not gates): printed in the terminal summary, so
# they show in quiet runs as well.
REPORTS: list[str] = []


@pytest.fixture
def report():
    return REPORTS.append


def pytest_terminal_summary(terminalreporter):
    if REPORTS:
        terminalreporter.section("reported figures")
        for line in REPORTS:
            terminalreporter.write_line(line)
