"""GPU parity of bd_select against the float64 oracle (HERALD Sec. IV-A2,
Sec. IV-B4).

* scores: the exported fp32 score vector against the oracle's float64
  scores, |g - r| <= 1e-4 |r| + 1e-6 max r;
* indices: bit-exact against the oracle's top-k run on the GPU's own fp32
  scores (the ranking decision is taken in fp32 on both sides), ties to the
  lower position, ascending, -1 padded.
"""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import check_scores, note
from oracle import bd_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


def _case(seed, B, S_list, Hq, Hkv, d=128, nq=32, C=None, dup=False):
    rs = np.random.default_rng(seed)
    C = C or max(S_list) + 16
    w = rs.standard_normal((B, 1, Hq, d)) / math.sqrt(d)
    Q = (w + 0.3 * rs.standard_normal((B, nq, Hq, d)) / math.sqrt(d)).astype(np.float32)
    K = rs.standard_normal((B, C, Hkv, d)).astype(np.float32) / math.sqrt(d)
    if dup:  # every key appears twice in a row: exact score ties
        K[:, 1::2] = K[:, 0:-1:2]
    return torch.from_numpy(Q).bfloat16(), torch.from_numpy(K).bfloat16()


def _run(bd, Q, K, s_len, k_sel, scale, mode=0, row=0, with_scores=True):
    B, Hkv = Q.shape[0], K.shape[2]
    s_max = max(int(max(s_len)), 1)
    k_max = max(int(max(k_sel)), 1)
    sc = torch.full((B, Hkv, s_max), -3.0, device="cuda") if with_scores else None
    idx = bd.select(Q.cuda(), K.cuda(), torch.tensor(s_len, dtype=torch.int32).cuda(), s_max,
                    torch.tensor(k_sel, dtype=torch.int32).cuda(), k_max, scale, rep_mode=mode,
                    rep_row=row, score_out=sc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (sc.cpu().double().numpy() if with_scores else None), k_max


def _check(Q, K, s_len, k_sel, scale, idx, sc, k_max, mode="mean", row=None, label=""):
    q_rep = orc.rep_query(Q, mode, row)
    ref, _, _ = orc.selection_scores(q_rep, K, s_len, scale)
    # rows with a zero budget are skipped: no scores are written for them
    scored = [int(S) if int(k) > 0 else 0 for S, k in zip(s_len, k_sel)]
    check_scores(sc, ref, scored, label)
    want = orc.topk_select(sc, s_len, k_sel, k_max)
    assert np.array_equal(idx, want), f"{label}: indices differ from the oracle top-k"
    return ref


@pytest.mark.parametrize("S_list,k_list,Hq,Hkv", [
    ([700, 0, 5000], [35, 10, 250], 8, 2),       # ragged, an empty row
    ([4096, 4097, 300], [205, 205, 300], 32, 8),  # chunk edges, k = S
    ([1000, 20], [1200, 50], 4, 4),               # k > S (G = 1)
    ([9000], [450], 16, 8),                       # G = 2
    ([2500, 2500], [125, 0], 64, 8),              # G = 8, k = 0 row
])
def test_select_small(bd, S_list, k_list, Hq, Hkv):
    note(f"select S={S_list} k={k_list} Hq={Hq} Hkv={Hkv}")
    B = len(S_list)
    Q, K = _case(sum(S_list), B, S_list, Hq, Hkv)
    scale = 1.0 / math.sqrt(128)
    idx, sc, k_max = _run(bd, Q, K, S_list, k_list, scale)
    _check(Q, K, S_list, k_list, scale, idx, sc, k_max, label="small")
    for b, (S, k) in enumerate(zip(S_list, k_list)):
        n = min(S, k)
        assert (idx[b, :, n:] == -1).all()
        if n:
            assert (np.diff(idx[b, :, :n], axis=1) > 0).all()


def test_select_row_mode(bd):
    note("select ROW mode (block centre)")
    Q, K = _case(5, 2, [3000, 1500], 32, 8)
    row = orc.center_row(32, 3000)
    idx, sc, k_max = _run(bd, Q, K, [3000, 1500], [150, 75], 0.088, mode=bd.BD_REP_ROW, row=row)
    _check(Q, K, [3000, 1500], [150, 75], 0.088, idx, sc, k_max, mode="row", row=row, label="row")


def test_select_exact_ties(bd):
    note("select with duplicated keys (exact ties)")
    S = [6000, 777]
    Q, K = _case(6, 2, S, 32, 8, dup=True)
    idx, sc, k_max = _run(bd, Q, K, S, [301, 39], 0.088)
    # ties are present at the threshold
    b, h = 0, 0
    kth = np.sort(sc[b, h, :S[b]])[::-1][300]
    assert (sc[b, h, :S[b]] == kth).sum() >= 2
    _check(Q, K, S, [301, 39], 0.088, idx, sc, k_max, label="ties")


def test_select_workspace_scores_and_determinism(bd):
    note("select: scores in workspace, run twice")
    S = [5000, 3000, 4096]
    Q, K = _case(7, 3, S, 32, 8)
    k = [250, 150, 205]
    idx1, sc1, _ = _run(bd, Q, K, S, k, 0.088)
    idx2, _, _ = _run(bd, Q, K, S, k, 0.088, with_scores=False)
    idx3, sc3, _ = _run(bd, Q, K, S, k, 0.088)
    assert np.array_equal(idx1, idx2) and np.array_equal(idx1, idx3)
    assert np.array_equal(sc1, sc3)


def test_planted_keys_recalled(bd):
    note("select: planted keys (reduced 32k workload)")
    wl = synth.sparse_32k(B=2, S=8192, T=1)
    idx, sc, k_max = _run(bd, wl.Qsel, wl.Kc, wl.s_len.tolist(), wl.k_sel.tolist(), wl.sm_scale)
    _check(wl.Qsel, wl.Kc, wl.s_len, wl.k_sel, wl.sm_scale, idx, sc, k_max, label="planted")
    for (b, h), pos in wl.planted.items():
        assert set(pos.tolist()) <= set(idx[b, h].tolist())


@pytest.mark.parametrize("S_list,k_list,dup", [
    ([40000, 33000, 5000], [2000, 40, 5000], False),   # multi-block ranking; k = S row
    ([36864, 100], [1843, 5], True),                   # exact ties at the threshold
])
def test_select_long_rows(bd, S_list, k_list, dup):
    """Rows longer than one block's LDS score cache: ranked by blocks of 4096
    scores (digit histograms in global memory, per-block counts, ordered
    write), ragged last blocks, a row whose budget covers its prefix."""
    note(f"select long rows S={S_list} k={k_list} dup={dup}")
    B = len(S_list)
    Q, K = _case(11 + int(dup), B, S_list, 16, 4, dup=dup)
    scale = 1.0 / math.sqrt(128)
    idx, sc, k_max = _run(bd, Q, K, S_list, k_list, scale)
    _check(Q, K, S_list, k_list, scale, idx, sc, k_max, label="long")
    for b, (S, k) in enumerate(zip(S_list, k_list)):
        n = min(S, k)
        assert (idx[b, :, n:] == -1).all()
        assert (np.diff(idx[b, :, :n], axis=1) > 0).all()
    if dup:
        kth = np.sort(sc[0, 0, :S_list[0]])[::-1][k_list[0] - 1]
        assert (sc[0, 0, :S_list[0]] == kth).sum() >= 2


@pytest.mark.parametrize("S_list,k_list,dup", [
    ([300000, 5000], [15000, 250], False),    # 74 blocks of 4096 scores on the long row
    ([270000], [13501], True),                # ... with exact ties at the threshold
])
def test_select_very_long_rows(bd, S_list, k_list, dup):
    """Rows of several hundred thousand scores (multi-block ranking with
    digit histograms in global memory, per-block counts, ordered write)."""
    note(f"select very long rows S={S_list} k={k_list} dup={dup}")
    B = len(S_list)
    Q, K = _case(21 + int(dup), B, S_list, 8, 2, dup=dup)
    scale = 1.0 / math.sqrt(128)
    idx, sc, k_max = _run(bd, Q, K, S_list, k_list, scale)
    _check(Q, K, S_list, k_list, scale, idx, sc, k_max, label="very long")
    for b, (S, k) in enumerate(zip(S_list, k_list)):
        n = min(S, k)
        assert (idx[b, :, n:] == -1).all()
        assert (np.diff(idx[b, :, :n], axis=1) > 0).all()


def test_select_all_scores_equal(bd):
    """Every key identical: every score ties at the threshold and the
    lowest positions are kept."""
    note("select: all scores equal")
    S_list, k_list = [20000, 3000], [1000, 2999]
    Q, K = _case(31, 2, S_list, 16, 4)
    K[:] = K[:, :1]
    idx, sc, k_max = _run(bd, Q, K, S_list, k_list, 0.088)
    for b, (S, k) in enumerate(zip(S_list, k_list)):
        assert (sc[b, :, :S] == sc[b, :, :1]).all()
        assert (idx[b, :, :k] == np.arange(k)).all() and (idx[b, :, k:] == -1).all()
    _check(Q, K, S_list, k_list, 0.088, idx, sc, k_max, label="all equal")
