"""Pins for the oracle's representative query, importance scores and top-k
(HERALD Sec. IV-A2 Eq. (2), Sec. IV-B4).
"""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch
import torch.nn.functional as F

import synth
from oracle import bd_oracle as orc


def test_center_row_eq2():
    """Eq. (2): for an even block the two middle positions tie; the oracle
    takes the later one, which is bl/2 (offsets to the block stay <= bl/2)."""
    assert orc.center_row(32, 100) == 16
    assert orc.center_row(8, 7) == 4
    assert orc.center_row(7, 50) == 3       # odd block: unique centre


def test_rep_query_modes():
    rs = np.random.default_rng(0)
    Q = rs.standard_normal((2, 5, 3, 4))
    np.testing.assert_allclose(orc.rep_query(Q, "mean"),
                               torch.from_numpy(Q).mean(1).numpy(), rtol=1e-15)
    np.testing.assert_array_equal(orc.rep_query(Q, "row", 2), Q[:, 2])
    same = np.repeat(Q[:, :1], 5, axis=1)
    np.testing.assert_allclose(orc.rep_query(same, "mean"), Q[:, 0], rtol=1e-15)


def _case(rs, B=2, S=50, Hq=8, Hkv=2, d=16, C=None):
    C = C or S + 4
    q_rep = rs.standard_normal((B, Hq, d))
    K = rs.standard_normal((B, C, Hkv, d))
    return q_rep, K


def test_scores_sum_to_G_and_attention_identity():
    """sum_s s_hat = G, and sum_s s_hat[s] V[s] equals the sum over the group
    of each head's softmax attention output (torch SDPA), because s_hat is
    the sum of the group's attention probabilities."""
    rs = np.random.default_rng(1)
    B, S, Hq, Hkv, d = 3, 77, 8, 2, 16
    G = Hq // Hkv
    q_rep, K = _case(rs, B, S, Hq, Hkv, d)
    V = rs.standard_normal(K.shape)
    s_len = np.array([S, 40, 1])
    sh, m, l = orc.selection_scores(q_rep, K, s_len, 0.7)
    for b in range(B):
        Sb = s_len[b]
        for h in range(Hkv):
            assert abs(sh[b, h, :Sb].sum() - G) < 1e-12
            assert (sh[b, h, Sb:] == 0).all()
            qt = torch.from_numpy(q_rep[b, h * G:(h + 1) * G])[:, None, :]   # [G, 1, d]
            kt = torch.from_numpy(K[b, :Sb, h])[None].expand(G, -1, -1)
            vt = torch.from_numpy(V[b, :Sb, h])[None].expand(G, -1, -1)
            att = F.scaled_dot_product_attention(qt, kt, vt, scale=0.7)[:, 0].sum(0).numpy()
            np.testing.assert_allclose(sh[b, h, :Sb] @ V[b, :Sb, h], att, rtol=1e-11, atol=1e-12)


def test_scores_g1_is_softmax():
    rs = np.random.default_rng(2)
    q_rep, K = _case(rs, B=1, S=31, Hq=3, Hkv=3, d=8)
    sh, _, _ = orc.selection_scores(q_rep, K, [31], 1.3)
    for h in range(3):
        z = 1.3 * (K[0, :31, h] @ q_rep[0, h])
        np.testing.assert_allclose(sh[0, h, :31], sps.softmax(z), rtol=1e-12)


def test_scores_s1_s2_closed_forms():
    rs = np.random.default_rng(3)
    q_rep, K = _case(rs, B=1, S=2, Hq=4, Hkv=1, d=8)
    sh, _, _ = orc.selection_scores(q_rep, K, [1], 0.5)
    assert abs(sh[0, 0, 0] - 4.0) < 1e-14
    sh, _, _ = orc.selection_scores(q_rep, K, [2], 0.5)
    dz = 0.5 * (q_rep[0] @ (K[0, 0, 0] - K[0, 1, 0]))      # z0 - z1 per head
    np.testing.assert_allclose(sh[0, 0, 0], sps.expit(dz).sum(), rtol=1e-13)
    np.testing.assert_allclose(sh[0, 0, 1], sps.expit(-dz).sum(), rtol=1e-13)


def test_scores_shift_invariance():
    """Adding one vector to every key shifts each head's logits by a
    constant, which the per-head softmax removes."""
    rs = np.random.default_rng(4)
    q_rep, K = _case(rs, B=1, S=60, Hq=8, Hkv=2, d=16)
    sh1, m1, _ = orc.selection_scores(q_rep, K, [60], 0.4)
    K2 = K + rs.standard_normal(16)[None, None, None, :] * 3.0
    sh2, m2, _ = orc.selection_scores(q_rep, K2, [60], 0.4)
    np.testing.assert_allclose(sh1, sh2, rtol=1e-10, atol=1e-14)
    assert not np.allclose(m1, m2)


def _brute_topk(sc, k):
    order = sorted(range(len(sc)), key=lambda s: (-sc[s], s))
    return sorted(order[:k])


@pytest.mark.parametrize("S,k,levels", [(8, 3, 3), (16, 5, 2), (64, 20, 5), (33, 33, 4),
                                        (40, 1, 1), (50, 17, 1000)])
def test_topk_bruteforce_with_ties(S, k, levels):
    rs = np.random.default_rng(S * 7 + k)
    sc = rs.integers(0, levels, size=(2, 3, S)).astype(np.float64) / 7.0
    idx = orc.topk_select(sc, [S, S], [k, k], k + 2)
    for b in range(2):
        for h in range(3):
            want = _brute_topk(list(sc[b, h]), k)
            assert list(idx[b, h, :k]) == want
            assert (idx[b, h, k:] == -1).all()


def test_topk_edge_budgets():
    sc = np.random.default_rng(5).random((3, 2, 10))
    idx = orc.topk_select(sc, [10, 4, 10], [12, 9, 0], 12)
    assert list(idx[0, 0, :10]) == list(range(10)) and (idx[0, :, 10:] == -1).all()
    assert list(idx[1, 1, :4]) == [0, 1, 2, 3] and (idx[1, :, 4:] == -1).all()
    assert (idx[2] == -1).all()


def test_budget_rounding():
    assert synth.budget_keys(32768, 0.05) == 1638
    assert synth.budget_keys(131072, 0.05) == 6554


def test_planted_keys_recalled():
    """Planted high-similarity keys (2 %) all land in the 5 % top-k."""
    wl = synth.sparse_32k(B=2, S=4096, T=1, Hq=8, Hkv=2, d=32)
    q_rep = orc.rep_query(wl.Qsel, "mean")
    sh, _, _ = orc.selection_scores(q_rep, wl.Kc, wl.s_len, wl.sm_scale)
    idx = orc.topk_select(sh, wl.s_len, wl.k_sel, wl.k_max)
    for (b, h), pos in wl.planted.items():
        sel = set(idx[b, h][idx[b, h] >= 0].tolist())
        assert set(pos.tolist()) <= sel
        # margin: every planted score beats every unplanted one
        mask = np.zeros(wl.s_max, bool)
        mask[pos] = True
        assert sh[b, h, mask].min() > sh[b, h, ~mask].max()


# ---------------------------------------------------------------------------
# exact multi-query selection (HERALD Sec. III-C, Sec. IV-A2 Fig. 8)
# ---------------------------------------------------------------------------

def _mq_case(rs, B=2, nq=5, S=40, Hq=8, Hkv=2, d=16):
    Q = rs.standard_normal((B, nq, Hq, d))
    K = rs.standard_normal((B, S + 3, Hkv, d))
    return Q, K


def test_multi_query_single_query_reduces_to_selection_scores():
    """nq = 1: exactly HERALD's single-query importance with that query."""
    rs = np.random.default_rng(11)
    Q, K = _mq_case(rs, B=2, nq=1, S=45)
    s_len = np.array([45, 17])
    got = orc.multi_query_scores(Q, K, s_len, 0.6)
    want, _, _ = orc.selection_scores(Q[:, 0], K, s_len, 0.6)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


def test_multi_query_sum_and_attention_identity():
    """sum_s s_hat = nq * G, and sum_s s_hat[s] V[s] equals the summed
    attention outputs of every (query, head) column (torch SDPA)."""
    rs = np.random.default_rng(12)
    B, nq, S, Hq, Hkv, d = 2, 6, 33, 8, 2, 16
    G = Hq // Hkv
    Q, K = _mq_case(rs, B, nq, S, Hq, Hkv, d)
    V = rs.standard_normal(K.shape)
    s_len = np.array([S, 9])
    sh = orc.multi_query_scores(Q, K, s_len, 0.45)
    for b in range(B):
        Sb = int(s_len[b])
        for h in range(Hkv):
            assert abs(sh[b, h, :Sb].sum() - nq * G) < 1e-11
            assert (sh[b, h, Sb:] == 0).all()
            qt = torch.from_numpy(Q[b, :, h * G:(h + 1) * G].reshape(nq * G, 1, d))
            kt = torch.from_numpy(K[b, :Sb, h])[None].expand(nq * G, -1, -1)
            vt = torch.from_numpy(V[b, :Sb, h])[None].expand(nq * G, -1, -1)
            att = F.scaled_dot_product_attention(qt, kt, vt, scale=0.45)[:, 0].sum(0).numpy()
            np.testing.assert_allclose(sh[b, h, :Sb] @ V[b, :Sb, h], att, rtol=1e-11, atol=1e-11)


def test_multi_query_identical_queries_and_permutation():
    """nq copies of one query give nq times its single-query scores (so the
    same ranking); reordering the queries changes nothing."""
    rs = np.random.default_rng(13)
    Q, K = _mq_case(rs, B=1, nq=4, S=50)
    same = np.repeat(Q[:, :1], 4, axis=1)
    one, _, _ = orc.selection_scores(Q[:, 0], K, [50], 0.3)
    np.testing.assert_allclose(orc.multi_query_scores(same, K, [50], 0.3), 4 * one, rtol=1e-12)
    base = orc.multi_query_scores(Q, K, [50], 0.3)
    perm = orc.multi_query_scores(Q[:, [2, 0, 3, 1]], K, [50], 0.3)
    np.testing.assert_allclose(perm, base, rtol=1e-12, atol=1e-15)


def test_multi_query_bruteforce_and_closed_forms():
    """Brute force with math.exp on a tiny case; S = 1 gives nq*G; S = 2 is a
    sum of logistic functions of the logit differences."""
    rs = np.random.default_rng(14)
    B, nq, S, Hq, Hkv, d = 1, 3, 6, 4, 2, 5
    G = Hq // Hkv
    Q, K = _mq_case(rs, B, nq, S, Hq, Hkv, d)
    sh = orc.multi_query_scores(Q, K, [S], 0.8)
    for h in range(Hkv):
        for s in range(S):
            tot = 0.0
            for i in range(nq):
                for g in range(G):
                    z = [0.8 * sum(Q[0, i, h * G + g, e] * K[0, u, h, e] for e in range(d)) for u in range(S)]
                    tot += math.exp(z[s]) / sum(math.exp(v) for v in z)
            assert abs(sh[0, h, s] - tot) < 1e-12
    sh1 = orc.multi_query_scores(Q, K, [1], 0.8)
    np.testing.assert_allclose(sh1[0, :, 0], nq * G, rtol=1e-15)
    sh2 = orc.multi_query_scores(Q, K, [2], 0.8)
    for h in range(Hkv):
        qc = Q[0, :, h * G:(h + 1) * G].reshape(-1, d)
        dz = 0.8 * (qc @ (K[0, 0, h] - K[0, 1, h]))
        np.testing.assert_allclose(sh2[0, h, 0], sps.expit(dz).sum(), rtol=1e-13)
        np.testing.assert_allclose(sh2[0, h, 1], sps.expit(-dz).sum(), rtol=1e-13)


def test_rep_attention_is_single_query_sdpa():
    """rep_attention against torch SDPA in float64, one query per head over
    the row's prefix; query head hq reads KV head hq // G; a row with no
    prefix gives zeros."""
    rs = np.random.default_rng(11)
    B, C, Hq, Hkv, d = 3, 70, 8, 2, 16
    G = Hq // Hkv
    q_rep = rs.standard_normal((B, Hq, d))
    K = rs.standard_normal((B, C, Hkv, d))
    V = rs.standard_normal((B, C, Hkv, d))
    s_len = np.array([70, 23, 0])
    o = orc.rep_attention(q_rep, K, V, s_len, 0.45)
    assert o.shape == (B, Hq, d)
    for b in range(B):
        S = int(s_len[b])
        for hq in range(Hq):
            if S == 0:
                assert (o[b, hq] == 0).all()
                continue
            h = hq // G
            qt = torch.from_numpy(q_rep[b, hq])[None, None]            # [1, 1, d]
            kt = torch.from_numpy(K[b, :S, h])[None]
            vt = torch.from_numpy(V[b, :S, h])[None]
            ref = F.scaled_dot_product_attention(qt, kt, vt, scale=0.45)[0, 0].numpy()
            np.testing.assert_allclose(o[b, hq], ref, rtol=1e-12, atol=1e-13)


def test_rep_attention_closed_forms():
    """Equal keys give the mean of the value rows; one prefix row gives that
    row; a key far more aligned with the query than the others gives its
    value row; the group's outputs summed equal s_hat @ V (the scores are the
    group's attention probabilities summed)."""
    rs = np.random.default_rng(12)
    Hq, Hkv, d, S = 4, 1, 8, 9
    q_rep = rs.standard_normal((1, Hq, d))
    V = rs.standard_normal((1, S, Hkv, d))
    K = np.repeat(rs.standard_normal((1, 1, Hkv, d)), S, axis=1)
    o = orc.rep_attention(q_rep, K, V, [S], 0.3)
    for hq in range(Hq):
        np.testing.assert_allclose(o[0, hq], V[0, :, 0].mean(0), rtol=1e-12, atol=1e-14)
    o1 = orc.rep_attention(q_rep, K, V, [1], 0.3)
    for hq in range(Hq):
        np.testing.assert_allclose(o1[0, hq], V[0, 0, 0], rtol=1e-14)
    K2 = rs.standard_normal((1, S, Hkv, d)) * 0.01
    K2[0, 5, 0] = 50.0 * q_rep[0, 2]
    o2 = orc.rep_attention(q_rep, K2, V, [S], 1.0)
    np.testing.assert_allclose(o2[0, 2], V[0, 5, 0], rtol=1e-9, atol=1e-9)
    K3 = rs.standard_normal((1, S, Hkv, d))
    o3 = orc.rep_attention(q_rep, K3, V, [S], 0.8)
    sh, _, _ = orc.selection_scores(q_rep, K3, [S], 0.8)
    np.testing.assert_allclose(o3[0].sum(0), sh[0, 0] @ V[0, :, 0], rtol=1e-12, atol=1e-13)
