"""Pins for the oracle's mask (FlowBlock review Eq. (6) / paper Eq. 5).

Each test checks ``oracle.eq6_mask`` against a formulation that is not the
Eq. (6) range test: block indices compared in logical sequence order (the
W-shaped block-causal rule the review states in words), the packing
diagram's worked rows, and the W = 1 and o_b = 0 special cases.
"""
import json
import os

import numpy as np
import pytest

from oracle import bd_oracle as orc


def _block_causal(C, q, bl, o, L):
    """Visibility from block indices: the prefix [0, o) holds committed blocks
    0..L-1, window slot s holds block L+s.  A query in block g sees a key in
    block g' iff g' <= g (W-shaped block-causal mask, bidirectional within a
    block).  Cache positions in [o, C-q) hold no block and are never seen."""
    t = C - q
    M = np.zeros((q, C), bool)
    for i in range(q):
        g = L + i // bl
        for j in range(C):
            if j < o:
                kb = j // bl
            elif j >= t:
                kb = L + (j - t) // bl
            else:
                continue
            M[i, j] = kb <= g
    return M


def test_hwp_diagram_rows(golden_dir):
    with open(os.path.join(golden_dir, "hwp_diagram.json")) as f:
        gd = json.load(f)
    bl, W, q = gd["bl"], gd["W"], gd["q"]
    assert q == W * bl
    C = 256
    o = np.array([s["o"] for s in gd["sequences"]])
    # the offset of a row is the start of its first active block: o = L * bl
    for s in gd["sequences"]:
        assert s["o"] == s["L"] * bl
        assert s["R"] - s["L"] <= W
    M = orc.eq6_mask(C, q, bl, o)
    for b, s in enumerate(gd["sequences"]):
        ref = _block_causal(C, q, bl, s["o"], s["L"])
        assert np.array_equal(M[b], ref)
        # slot 0 sees prefix + one block, slot 1 sees prefix + two blocks
        counts = M[b].sum(axis=1)
        assert np.array_equal(counts[:bl], np.full(bl, s["o"] + bl))
        assert np.array_equal(counts[bl:], np.full(bl, s["o"] + 2 * bl))


@pytest.mark.parametrize("bl,W,C", [(4, 3, 40), (8, 2, 64), (5, 4, 61), (16, 1, 48)])
def test_mask_block_causal_bruteforce(bl, W, C):
    q = W * bl
    t = C - q
    rs = np.random.default_rng(bl * 100 + W)
    # offsets at block starts (the committed prefix holds whole blocks)
    Ls = [0, 1, t // bl] + list(rs.integers(0, t // bl + 1, size=4))
    o = np.array([L * bl for L in Ls])
    M = orc.eq6_mask(C, q, bl, o)
    for b, L in enumerate(Ls):
        assert np.array_equal(M[b], _block_causal(C, q, bl, o[b], L))


def test_mask_w1_is_block_causal_denoising():
    """W = 1: every query sees the whole prefix and its whole block, nothing
    else (HERALD Sec. II-A: bidirectional in-block, causal to the cache)."""
    C, bl = 96, 16
    o = np.array([0, 16, 48, 80])
    M = orc.eq6_mask(C, bl, bl, o)
    t = C - bl
    for b, ob in enumerate(o):
        want = np.zeros(C, bool)
        want[:ob] = True
        want[t:] = True
        assert (M[b] == want[None, :]).all()


def test_mask_zero_offset_window_only():
    C, bl, W = 128, 8, 4
    q = W * bl
    M = orc.eq6_mask(C, q, bl, np.array([0]))[0]
    assert not M[:, :C - q].any()
    # lower block-triangular over the window, with full bl x bl diagonal blocks
    win = M[:, C - q:]
    for i in range(q):
        assert win[i].sum() == (i // bl + 1) * bl
        assert win[i, :(i // bl + 1) * bl].all()


def test_mask_unaligned_offsets():
    """Offsets need not sit at block starts: the prefix part is the plain
    range [0, o_b)."""
    C, bl, W = 100, 8, 2
    q = W * bl
    o = np.array([3, 37, 84])
    M = orc.eq6_mask(C, q, bl, o)
    for b, ob in enumerate(o):
        assert M[b][:, :ob].all()
        assert not M[b][:, ob:C - q].any()


def test_window_visible_matches_eq6_tail():
    for bl, W in [(32, 2), (7, 3), (1, 5)]:
        q = W * bl
        C = q + 10
        M = orc.eq6_mask(C, q, bl, np.array([0]))[0]
        assert np.array_equal(orc.window_visible(q, bl), M[:, C - q:])


# ---------------------------------------------------------------------------
# the two other window masks: HERALD's isolated draft/denoise groups (Sec.
# IV-B2) and Flash-dLLM's verify views (block 0 shared)
# ---------------------------------------------------------------------------

def _groups_by_rule(q, bl, mode):
    """Enumerate (query group, key group) pairs in words: isolated groups see
    only themselves; with a shared first group every group also sees group
    0, and group 0 sees only itself."""
    M = np.zeros((q, q), bool)
    for i in range(q):
        for w in range(q):
            gi, gw = i // bl, w // bl
            if mode == "isolated":
                M[i, w] = gi == gw
            else:
                M[i, w] = gi == gw or gw == 0
    return M


@pytest.mark.parametrize("mode", ["isolated", "shared_first"])
@pytest.mark.parametrize("q,bl", [(64, 32), (96, 32), (12, 4), (5, 5)])
def test_other_window_modes_by_rule(mode, q, bl):
    np.testing.assert_array_equal(orc.window_visible(q, bl, mode), _groups_by_rule(q, bl, mode))


def test_other_modes_special_cases():
    # one block: every mode is plain bidirectional attention over the block
    for mode in orc.MASK_MODES:
        assert orc.window_visible(32, 32, mode).all()
    # two blocks: the shared-first views equal the block-causal mask
    np.testing.assert_array_equal(orc.window_visible(64, 32, "shared_first"),
                                  orc.window_visible(64, 32, "block_causal"))
    # isolated is block-diagonal: its complement within block-causal is the strict lower blocks
    bc, iso = orc.window_visible(96, 32, "block_causal"), orc.window_visible(96, 32, "isolated")
    assert (iso <= bc).all() and iso.sum() == 3 * 32 * 32
    with pytest.raises(ValueError):
        orc.window_visible(64, 32, "causal")


@pytest.mark.parametrize("mode", ["isolated", "shared_first"])
def test_cache_mask_other_modes(mode):
    """In the cache form the prefix part is unchanged and the tail carries
    the window mode; rows [o_b, t) stay invisible."""
    C, q, bl = 200, 96, 32
    t = C - q
    o = np.array([0, 40, t])
    M = orc.eq6_mask(C, q, bl, o, mode)
    W = _groups_by_rule(q, bl, mode)
    for b, ob in enumerate(o):
        assert M[b][:, :ob].all() and not M[b][:, ob:t].any()
        np.testing.assert_array_equal(M[b][:, t:], W)
