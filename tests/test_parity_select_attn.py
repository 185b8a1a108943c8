"""GPU parity of bd_select_attn: the representative query's attention output
over the full prefix beside the selection (HERALD Sec. IV-B4), against the
float64 oracle's ``rep_attention``.

* o_rep: bf16 outputs within |g - r| <= 2e-2 + 1e-2 |r| elementwise, and a
  tighter bound on the largest error relative to the largest output of the
  (row, query head), max |g - r| <= 4e-3 max |r| + 1e-5 (bf16 rounding of
  the output is 2^-9 relative);
* rows with no prefix or no budget: o_rep exactly zero;
* the selection itself: indices and exported scores bit-identical to
  bd_select on the same inputs (the same kernels rank them).
"""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import note
from oracle import bd_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


def _case(seed, B, S_list, Hq, Hkv, d=128, nq=32, C=None, peaky=False):
    rs = np.random.default_rng(seed)
    C = C or max(S_list) + 16
    w = rs.standard_normal((B, 1, Hq, d)) / math.sqrt(d)
    Q = (w + 0.3 * rs.standard_normal((B, nq, Hq, d)) / math.sqrt(d)).astype(np.float32)
    K = rs.standard_normal((B, C, Hkv, d)).astype(np.float32) / math.sqrt(d)
    V = rs.standard_normal((B, C, Hkv, d)).astype(np.float32)
    if peaky:   # a few keys aligned with the group's mean query: a sharp softmax
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hkv):
                qm = w[b, 0, h * G:(h + 1) * G].mean(0)
                for s in rs.choice(min(S_list[b], C) or 1, size=3, replace=False):
                    K[b, s, h] = 6.0 * qm / np.linalg.norm(qm)
    return (torch.from_numpy(Q).bfloat16(), torch.from_numpy(K).bfloat16(),
            torch.from_numpy(V).bfloat16())


def _check_out(o_gpu, ref, S_list, k_list, label):
    g = o_gpu.detach().cpu().double().numpy()
    assert np.isfinite(g).all(), f"{label}: non-finite o_rep"
    for b, (S, k) in enumerate(zip(S_list, k_list)):
        if S == 0 or k == 0:
            assert (g[b] == 0).all(), f"{label}: row {b} without prefix or budget is not zero"
            continue
        err = np.abs(g[b] - ref[b])
        assert (err <= 2e-2 + 1e-2 * np.abs(ref[b])).all(), f"{label}: row {b} max err {err.max():.3e}"
        for hq in range(g.shape[1]):
            bound = 4e-3 * np.abs(ref[b, hq]).max() + 1e-5
            assert err[hq].max() <= bound, (f"{label}: row {b} head {hq}: max err {err[hq].max():.3e} "
                                            f"vs bound {bound:.3e}")


def _run(bd, Q, K, V, s_len, k_sel, scale, mode=0, row=0):
    B, Hkv = Q.shape[0], K.shape[2]
    s_max = max(int(max(s_len)), 1)
    k_max = max(int(max(k_sel)), 1)
    sl = torch.tensor(s_len, dtype=torch.int32).cuda()
    ks = torch.tensor(k_sel, dtype=torch.int32).cuda()
    Qc, Kc, Vc = Q.cuda(), K.cuda(), V.cuda()
    sc_a = torch.full((B, Hkv, s_max), -3.0, device="cuda")
    sc_s = torch.full((B, Hkv, s_max), -3.0, device="cuda")
    o_rep = torch.full((B, Q.shape[2], Q.shape[3]), float("nan"), dtype=torch.bfloat16, device="cuda")
    idx_a, o_rep = bd.select_attn(Qc, Kc, Vc, sl, s_max, ks, k_max, scale, rep_mode=mode, rep_row=row,
                                  score_out=sc_a, o_rep=o_rep)
    idx_s = bd.select(Qc, Kc, sl, s_max, ks, k_max, scale, rep_mode=mode, rep_row=row, score_out=sc_s)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_s), "indices differ from bd_select's"
    assert torch.equal(sc_a, sc_s), "scores differ from bd_select's"
    return o_rep


@pytest.mark.parametrize("S_list,k_list,Hq,Hkv,peaky", [
    ([700, 0, 5000], [35, 10, 250], 8, 2, False),         # ragged, an empty row
    ([1023, 1024, 1025], [50, 0, 1025], 32, 8, False),    # chunk edges, k = 0 and k = S rows
    ([2049, 20], [1200, 50], 4, 4, True),                 # k > S, G = 1, sharp softmax
    ([9000], [450], 16, 8, True),                         # G = 2
    ([2500, 3100], [125, 155], 64, 8, False),             # G = 8
])
def test_select_attn_small(bd, S_list, k_list, Hq, Hkv, peaky):
    note(f"select_attn S={S_list} k={k_list} Hq={Hq} Hkv={Hkv} peaky={peaky}")
    Q, K, V = _case(sum(S_list) + Hq, len(S_list), S_list, Hq, Hkv, peaky=peaky)
    scale = 1.0 / math.sqrt(128)
    o_rep = _run(bd, Q, K, V, S_list, k_list, scale)
    ref = orc.rep_attention(orc.rep_query(Q, "mean"), K, V, S_list, scale)
    _check_out(o_rep, ref, S_list, k_list, "small")


def test_select_attn_row_mode_and_long_row(bd):
    """One query row as the representative; a 40,000-position row (40 output
    chunks, the multi-block ranking path) beside a short one."""
    S_list, k_list = [40000, 1500], [2000, 75]
    note(f"select_attn ROW mode S={S_list}")
    Q, K, V = _case(7, 2, S_list, 32, 8, peaky=True)
    row = orc.center_row(32, 40000)
    o_rep = _run(bd, Q, K, V, S_list, k_list, 0.088, mode=bd.BD_REP_ROW, row=row)
    ref = orc.rep_attention(orc.rep_query(Q, "row", row), K, V, S_list, 0.088)
    _check_out(o_rep, ref, S_list, k_list, "row/long")


def test_select_attn_zero_budget_everywhere(bd):
    """k_max = 0: nothing is selected and every output row is zero."""
    note("select_attn k_max = 0")
    Q, K, V = _case(3, 2, [300, 200], 8, 2)
    o_rep = torch.full((2, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    bd.select_attn(Q.cuda(), K.cuda(), V.cuda(), torch.tensor([300, 200], dtype=torch.int32).cuda(), 300,
                   torch.zeros(2, dtype=torch.int32).cuda(), 0, 0.088, o_rep=o_rep)
    torch.cuda.synchronize()
    assert (o_rep == 0).all()


@pytest.mark.parametrize("name", ["sparse_32k", "sparse_128k"])
def test_select_attn_configs(bd, name):
    """The sparse workloads at full size (4 x 32K rows, one 128K row; planted
    high-similarity keys), every row and query head against the oracle."""
    note(f"select_attn config {name}")
    wl = getattr(synth, name)()
    o_rep = _run(bd, wl.Qsel, wl.Kc, wl.Vc, [int(x) for x in wl.s_len], [int(x) for x in wl.k_sel],
                 wl.sm_scale)
    ref = orc.rep_attention(orc.rep_query(wl.Qsel, "mean"), wl.Kc, wl.Vc, wl.s_len, wl.sm_scale)
    _check_out(o_rep, ref, [int(x) for x in wl.s_len], [int(x) for x in wl.k_sel], name)


def test_select_attn_graph_replay(bd):
    """Captured in a HIP graph and replayed three times, with eager calls on
    other inputs in between: indices and outputs equal the eager call's (the
    workspace's histograms are cleared by a kernel, not a memset)."""
    note("select_attn graph replay")
    S_list, k_list = [3000, 1200], [150, 60]
    Q, K, V = (t.cuda() for t in _case(21, 2, S_list, 32, 8, peaky=True))
    Q2, K2, V2 = (t.cuda() for t in _case(22, 2, S_list, 32, 8))
    sl = torch.tensor(S_list, dtype=torch.int32).cuda()
    ks = torch.tensor(k_list, dtype=torch.int32).cuda()
    idx = torch.empty((2, 8, 150), dtype=torch.int32, device="cuda")
    o_rep = torch.empty((2, 32, 128), dtype=torch.bfloat16, device="cuda")
    ws = bd.workspace(bd.select_attn_workspace_size(2, 32, 8, 128, 3000, 150), "cuda")

    def call():
        bd.select_attn(Q, K, V, sl, 3000, ks, 150, 0.088, idx_out=idx, o_rep=o_rep, ws=ws)
    call()
    torch.cuda.synchronize()
    want_idx, want_o = idx.clone(), o_rep.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        bd.select_attn(Q2, K2, V2, sl, 3000, ks, 150, 0.088, idx_out=idx, o_rep=o_rep, ws=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want_idx), f"replay {rep}: indices"
        assert torch.equal(o_rep, want_o), f"replay {rep}: o_rep"
