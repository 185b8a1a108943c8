"""Shared helpers of the GPU parity tests."""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {torch.bfloat16: (2e-2, 1e-2, 1e-2), torch.float32: (1e-4, 1e-4, 1e-5)}


def note(msg: str):
    """Name the case before a GPU step (kept visible if the step dies)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy()
    return t.view(torch.int32).numpy()


def check_attention(out_gpu: torch.Tensor, ref: np.ndarray, dtype, rows=None, label=""):
    """Elementwise |g - r| <= atol + rtol*|r| and, per (row, query head), the
    normalised error ||g - r|| / ||r|| over (query, d) below the stated bound."""
    atol, rtol, nrm = TOL[dtype]
    g = out_gpu.detach().cpu().double().numpy()
    rows = range(g.shape[0]) if rows is None else [int(r) for r in rows]
    worst = 0.0
    worst_n = 0.0
    for b in rows:
        gb, rb = g[b], ref[b]
        assert np.isfinite(gb).all(), f"{label}: non-finite output in row {b}"
        err = np.abs(gb - rb)
        bad = err > atol + rtol * np.abs(rb)
        assert not bad.any(), (f"{label}: row {b}: {bad.sum()} elements out of tolerance, "
                               f"max err {err.max():.3e}")
        num = np.sqrt(((gb - rb) ** 2).sum(axis=(0, 2)))
        den = np.sqrt((rb ** 2).sum(axis=(0, 2)))
        ne = (num / np.maximum(den, 1e-30)).max()
        assert ne <= nrm, f"{label}: row {b}: normalised error {ne:.3e} > {nrm}"
        worst = max(worst, err.max())
        worst_n = max(worst_n, ne)
    return worst, worst_n


def check_scores(sc_gpu: np.ndarray, sc_ref: np.ndarray, s_len, label=""):
    """|g - r| <= 1e-4 |r| + 1e-6 max(r) per (row, KV head) over s < S_b."""
    for b in range(sc_ref.shape[0]):
        S = int(s_len[b])
        if S == 0:
            continue
        for h in range(sc_ref.shape[1]):
            r = sc_ref[b, h, :S]
            g = sc_gpu[b, h, :S]
            bound = 1e-4 * np.abs(r) + 1e-6 * r.max()
            err = np.abs(g - r)
            assert (err <= bound).all(), (f"{label}: scores of row {b} head {h}: max rel err "
                                          f"{(err / np.maximum(np.abs(r), 1e-30)).max():.3e}")
