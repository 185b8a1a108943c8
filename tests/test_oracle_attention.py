"""Pins for the oracle's block-diffusion attention.

``oracle.block_attention`` / ``oracle.cache_attention_eq6`` are checked
against torch's scaled_dot_product_attention (float64, CPU) with an
explicit boolean mask, closed forms (constant V, equal logits, one-hot
logits), invariances (pool order, G = 1), and the FlowBlock review's "free
retire" property.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import bd_oracle as orc


def _rand(rs, *shape, scale=1.0):
    return rs.standard_normal(shape) * scale


def _sdpa(Q, keys, vals, mask, scale):
    """torch SDPA in float64 on the CPU.  Q [q, Hq, d], keys/vals [n, Hkv, d],
    mask [q, n] (True = attend).  GQA by repeating each KV head G times."""
    q, Hq, d = Q.shape
    Hkv = keys.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(Q).permute(1, 0, 2)[None]                 # [1, Hq, q, d]
    kt = torch.from_numpy(keys).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(vals).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                         scale=scale)
    return out[0].permute(1, 0, 2).numpy()                           # [q, Hq, d]


@pytest.mark.parametrize("B,Hq,Hkv,d,bl,W,P", [
    (3, 4, 1, 16, 8, 2, 37),
    (2, 8, 2, 32, 4, 3, 5),
    (2, 4, 4, 8, 16, 1, 64),
    (1, 6, 3, 16, 5, 4, 0),
])
def test_block_attention_vs_sdpa(B, Hq, Hkv, d, bl, W, P):
    rs = np.random.default_rng(B * 1000 + Hq * 10 + d)
    q = W * bl
    sc = 1.0 / math.sqrt(d)
    Q = _rand(rs, B, q, Hq, d)
    PK, PV = _rand(rs, B, P + 3, Hkv, d), _rand(rs, B, P + 3, Hkv, d)
    WK, WV = _rand(rs, B, q, Hkv, d), _rand(rs, B, q, Hkv, d)
    p_len = rs.integers(0, P + 1, size=B)
    p_len[0] = P
    O, LSE = orc.block_attention(Q, PK, PV, p_len, WK, WV, bl, sc)
    for b in range(B):
        Pb = int(p_len[b])
        keys = np.concatenate([PK[b, :Pb], WK[b]], 0)
        vals = np.concatenate([PV[b, :Pb], WV[b]], 0)
        mask = np.zeros((q, Pb + q), bool)
        mask[:, :Pb] = True
        for i in range(q):
            mask[i, Pb:Pb + (i // bl + 1) * bl] = True
        ref = _sdpa(Q[b], keys, vals, mask, sc)
        np.testing.assert_allclose(O[b], ref, rtol=1e-12, atol=1e-12)
        # LSE against torch.logsumexp over the visible logits
        G = Hq // Hkv
        for hq in range(Hq):
            lg = torch.from_numpy(sc * Q[b, :, hq] @ keys[:, hq // G].T)
            lg = lg.masked_fill(~torch.from_numpy(mask), -math.inf)
            np.testing.assert_allclose(LSE[b, hq], torch.logsumexp(lg, -1).numpy(),
                                       rtol=1e-12, atol=1e-12)


def test_cache_form_vs_sdpa_with_nan_sentinels():
    """Eq. (6) over a cache whose invisible rows [o_b, t) hold NaN."""
    rs = np.random.default_rng(7)
    B, C, Hq, Hkv, d, bl, W = 3, 96, 4, 2, 16, 8, 2
    q = W * bl
    t = C - q
    o = np.array([0, 24, 80])
    Kc, Vc = _rand(rs, B, C, Hkv, d), _rand(rs, B, C, Hkv, d)
    for b in range(B):
        Kc[b, o[b]:t] = np.nan
        Vc[b, o[b]:t] = np.nan
    Q = _rand(rs, B, q, Hq, d)
    O, _ = orc.cache_attention_eq6(Q, Kc, Vc, o, bl, 0.25)
    assert np.isfinite(O).all()
    M = orc.eq6_mask(C, q, bl, o)
    for b in range(B):
        cols = np.nonzero(M[b].any(0))[0]
        ref = _sdpa(Q[b], Kc[b, cols], Vc[b, cols], M[b][:, cols], 0.25)
        np.testing.assert_allclose(O[b], ref, rtol=1e-12, atol=1e-12)


def test_cache_form_equals_prefix_window_form():
    rs = np.random.default_rng(8)
    B, C, Hq, Hkv, d, bl, W = 2, 80, 8, 2, 8, 4, 3
    q = W * bl
    t = C - q
    o = np.array([5, t])
    Kc, Vc = _rand(rs, B, C, Hkv, d), _rand(rs, B, C, Hkv, d)
    Q = _rand(rs, B, q, Hq, d)
    O1, L1 = orc.cache_attention_eq6(Q, Kc, Vc, o, bl, 0.3)
    O2, L2 = orc.block_attention(Q, Kc, Vc, o, Kc[:, t:], Vc[:, t:], bl, 0.3)
    np.testing.assert_allclose(O1, O2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=1e-13, atol=1e-13)


def test_w1_zero_prefix_is_plain_bidirectional_sdpa():
    rs = np.random.default_rng(9)
    bl, Hq, d = 16, 2, 8
    Q = _rand(rs, 1, bl, Hq, d)
    WK, WV = _rand(rs, 1, bl, Hq, d), _rand(rs, 1, bl, Hq, d)
    O, _ = orc.block_attention(Q, WK[:, :0], WV[:, :0], [0], WK, WV, bl, 0.5)
    qt = torch.from_numpy(Q[0]).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(qt, torch.from_numpy(WK[0]).permute(1, 0, 2),
                                         torch.from_numpy(WV[0]).permute(1, 0, 2), scale=0.5)
    np.testing.assert_allclose(O[0], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_equal_logits_closed_form():
    """Q = 0: all visible logits are 0, so O is the mean of the visible V
    rows and LSE = log(#visible) = log(P_b + (floor(i/bl)+1)*bl)."""
    rs = np.random.default_rng(10)
    B, Hq, Hkv, d, bl, W, P = 2, 4, 2, 8, 4, 3, 11
    q = W * bl
    Q = np.zeros((B, q, Hq, d))
    PK, PV = _rand(rs, B, P, Hkv, d), _rand(rs, B, P, Hkv, d)
    WK, WV = _rand(rs, B, q, Hkv, d), _rand(rs, B, q, Hkv, d)
    p_len = np.array([P, 3])
    O, LSE = orc.block_attention(Q, PK, PV, p_len, WK, WV, bl, 1.0)
    for b in range(B):
        for i in range(q):
            nw = (i // bl + 1) * bl
            for hq in range(Hq):
                h = hq // (Hq // Hkv)
                want = np.concatenate([PV[b, :p_len[b], h], WV[b, :nw, h]]).mean(0)
                np.testing.assert_allclose(O[b, i, hq], want, rtol=1e-13, atol=1e-13)
                assert abs(LSE[b, hq, i] - math.log(p_len[b] + nw)) < 1e-13


def test_constant_v_and_one_hot_logits():
    rs = np.random.default_rng(11)
    B, Hq, Hkv, d, bl, W, P = 1, 2, 1, 8, 4, 2, 9
    q = W * bl
    Q = _rand(rs, B, q, Hq, d)
    PK = _rand(rs, B, P, Hkv, d)
    WK = _rand(rs, B, q, Hkv, d)
    # constant V -> constant O
    PV = np.full((B, P, Hkv, d), 3.25)
    WV = np.full((B, q, Hkv, d), 3.25)
    O, _ = orc.block_attention(Q, PK, PV, [P], WK, WV, bl, 0.5)
    np.testing.assert_allclose(O, 3.25, rtol=1e-14)
    # one-hot: key 4 of the prefix aligned with every query, others orthogonal
    Q = np.zeros((B, q, Hq, d))
    Q[..., 0] = 1.0
    PK = np.zeros((B, P, Hkv, d))
    PK[0, 4, 0, 0] = 1000.0
    WK = np.zeros((B, q, Hkv, d))
    PV, WV = _rand(rs, B, P, Hkv, d), _rand(rs, B, q, Hkv, d)
    O, _ = orc.block_attention(Q, PK, PV, [P], WK, WV, bl, 1.0)
    np.testing.assert_allclose(O[0], np.broadcast_to(PV[0, 4, 0], O[0].shape), rtol=1e-12)


def test_pool_order_invariance_and_g1():
    rs = np.random.default_rng(12)
    B, Hq, Hkv, d, bl, W, P = 2, 4, 4, 8, 4, 2, 13
    q = W * bl
    Q = _rand(rs, B, q, Hq, d)
    PK, PV = _rand(rs, B, P, Hkv, d), _rand(rs, B, P, Hkv, d)
    WK, WV = _rand(rs, B, q, Hkv, d), _rand(rs, B, q, Hkv, d)
    O1, L1 = orc.block_attention(Q, PK, PV, [P, P], WK, WV, bl, 0.4)
    perm = rs.permutation(P)
    O2, L2 = orc.block_attention(Q, PK[:, perm], PV[:, perm], [P, P], WK, WV, bl, 0.4)
    np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=1e-13)
    # G = 1 per head equals running each head alone
    for hq in range(Hq):
        Oh, _ = orc.block_attention(Q[:, :, hq:hq + 1], PK[:, :, hq:hq + 1], PV[:, :, hq:hq + 1],
                                    [P, P], WK[:, :, hq:hq + 1], WV[:, :, hq:hq + 1], bl, 0.4)
        np.testing.assert_allclose(Oh[:, :, 0], O1[:, :, hq], rtol=1e-13, atol=1e-14)


def test_full_budget_pool_equals_dense_cache():
    """A 100 % budget (pool = the whole prefix, in order) is dense attention."""
    rs = np.random.default_rng(13)
    B, C, Hq, Hkv, d, bl, W = 2, 64, 4, 2, 8, 8, 2
    q = W * bl
    t = C - q
    o = np.array([20, 48])
    Kc, Vc = _rand(rs, B, C, Hkv, d), _rand(rs, B, C, Hkv, d)
    Q = _rand(rs, B, q, Hq, d)
    Od, _ = orc.cache_attention_eq6(Q, Kc, Vc, o, bl, 0.3)
    idx = np.full((B, Hkv, t), -1)
    for b in range(B):
        idx[b, :, :o[b]] = np.arange(o[b])
    pool_k = orc.gather(Kc, idx, o, np.zeros((B, t, Hkv, d)))
    pool_v = orc.gather(Vc, idx, o, np.zeros((B, t, Hkv, d)))
    Op, _ = orc.block_attention(Q, pool_k, pool_v, o, Kc[:, t:], Vc[:, t:], bl, 0.3)
    np.testing.assert_allclose(Od, Op, rtol=1e-13, atol=1e-13)


def test_free_retire_shift_equivalence():
    """FlowBlock review Sec. 5 ("free retire"): after the scatter-back of
    Eq. (7), retiring the first window block is only o_b += bl.  A query of
    old slot 1 and the same query in new slot 0 see the same key set, so
    their outputs agree."""
    rs = np.random.default_rng(14)
    B, C, Hq, Hkv, d, bl, W = 1, 128, 4, 2, 8, 8, 2
    q = W * bl
    t = C - q
    o = np.array([40])
    Kc, Vc = _rand(rs, B, C, Hkv, d), _rand(rs, B, C, Hkv, d)
    Kc[0, o[0]:t] = np.nan
    Vc[0, o[0]:t] = np.nan
    Q = _rand(rs, B, q, Hq, d)
    O_before, _ = orc.cache_attention_eq6(Q, Kc, Vc, o, bl, 0.35)
    # scatter the window into place (one layer), retire block 0
    K2 = orc.kv_scatter(Kc[None], Kc[None], o, t, q)[0]
    V2 = orc.kv_scatter(Vc[None], Vc[None], o, t, q)[0]
    o2 = o + bl
    # old slot 1 moves to new slot 0 at the tail; new slot 1 gets fresh KV
    K2[0, t:t + bl] = Kc[0, t + bl:]
    V2[0, t:t + bl] = Vc[0, t + bl:]
    K2[0, t + bl:] = _rand(rs, bl, Hkv, d)
    V2[0, t + bl:] = _rand(rs, bl, Hkv, d)
    Q2 = np.concatenate([Q[:, bl:], _rand(rs, B, bl, Hq, d)], axis=1)
    O_after, _ = orc.cache_attention_eq6(Q2, K2, V2, o2, bl, 0.35)
    np.testing.assert_allclose(O_after[:, :bl], O_before[:, bl:], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# window mask modes (HERALD Sec. IV-B2 isolated groups; Flash-dLLM verify
# views with a shared first block)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["isolated", "shared_first"])
def test_mode_attention_vs_sdpa(mode):
    rs = np.random.default_rng(31)
    B, Hq, Hkv, d, bl, W, P = 2, 8, 2, 16, 4, 3, 9
    q = W * bl
    Q = _rand(rs, B, q, Hq, d)
    PK, PV = _rand(rs, B, P, Hkv, d), _rand(rs, B, P, Hkv, d)
    WK, WV = _rand(rs, B, q, Hkv, d), _rand(rs, B, q, Hkv, d)
    p_len = np.array([P, 0])
    O, _ = orc.block_attention(Q, PK, PV, p_len, WK, WV, bl, 0.3, mode=mode)
    for b in range(B):
        Pb = int(p_len[b])
        keys = np.concatenate([PK[b, :Pb], WK[b]], 0)
        vals = np.concatenate([PV[b, :Pb], WV[b]], 0)
        mask = np.zeros((q, Pb + q), bool)
        mask[:, :Pb] = True
        for i in range(q):
            g = i // bl
            mask[i, Pb + g * bl:Pb + (g + 1) * bl] = True
            if mode == "shared_first":
                mask[i, Pb:Pb + bl] = True
        np.testing.assert_allclose(O[b], _sdpa(Q[b], keys, vals, mask, 0.3), rtol=1e-12, atol=1e-12)


def test_isolated_groups_equal_separate_forwards():
    """HERALD's fused draft/denoise forward: each group's output equals a
    forward of that group alone (W = 1) over the same prefix."""
    rs = np.random.default_rng(32)
    B, Hq, Hkv, d, bl, W, P = 2, 4, 2, 8, 8, 2, 13
    q = W * bl
    Q = _rand(rs, B, q, Hq, d)
    PK, PV = _rand(rs, B, P, Hkv, d), _rand(rs, B, P, Hkv, d)
    WK, WV = _rand(rs, B, q, Hkv, d), _rand(rs, B, q, Hkv, d)
    p_len = np.array([P, 5])
    O, L = orc.block_attention(Q, PK, PV, p_len, WK, WV, bl, 0.4, mode="isolated")
    for g in range(W):
        sl = slice(g * bl, (g + 1) * bl)
        Og, Lg = orc.block_attention(Q[:, sl], PK, PV, p_len, WK[:, sl], WV[:, sl], bl, 0.4)
        np.testing.assert_allclose(O[:, sl], Og, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(L[:, :, sl], Lg, rtol=1e-13, atol=1e-14)


def test_shared_first_views_equal_two_block_forwards():
    """Each view block j >= 1 gives what the block-causal W = 2 forward of
    (block 0, block j) gives for its second block; block 0 what it gives alone."""
    rs = np.random.default_rng(33)
    B, Hq, Hkv, d, bl, W, P = 1, 4, 1, 8, 4, 4, 6
    q = W * bl
    Q = _rand(rs, B, q, Hq, d)
    PK, PV = _rand(rs, B, P, Hkv, d), _rand(rs, B, P, Hkv, d)
    WK, WV = _rand(rs, B, q, Hkv, d), _rand(rs, B, q, Hkv, d)
    p_len = np.array([P])
    O, _ = orc.block_attention(Q, PK, PV, p_len, WK, WV, bl, 0.5, mode="shared_first")
    O0, _ = orc.block_attention(Q[:, :bl], PK, PV, p_len, WK[:, :bl], WV[:, :bl], bl, 0.5)
    np.testing.assert_allclose(O[:, :bl], O0, rtol=1e-13, atol=1e-14)
    for j in range(1, W):
        idx = np.r_[0:bl, j * bl:(j + 1) * bl]
        Oj, _ = orc.block_attention(Q[:, idx], PK, PV, p_len, WK[:, idx], WV[:, idx], bl, 0.5)
        np.testing.assert_allclose(O[:, j * bl:(j + 1) * bl], Oj[:, bl:], rtol=1e-13, atol=1e-14)
