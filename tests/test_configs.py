"""GPU parity at the full sizes of the five synthetic workloads, in the
launch configuration the benchmark times (``BlockDiffusionStep``).

Indices, gathers and scatters are compared bit-exactly; scores and
attention outputs within the stated tolerances.  Where the float64 oracle
would take too long (dense attention of the 64-row serving mix), a sample
of rows is checked one by one; everything else is checked in full.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import bits, check_attention, check_scores, note
from oracle import bd_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


def _dev(wl):
    return wl.Kc.cuda(), wl.Vc.cuda(), wl.Q.cuda(), wl.o.cuda()


def test_packed_wavefront_config(bd):
    """8 rows, C = 4096, W = 2, o_b multiples of 32 in [512, 3968]: W-shaped
    attention over each row's own prefix + window, then the scatter-back."""
    from sparse_kv_cache_bd_amd.pipeline import BlockDiffusionStep
    note("config packed_wavefront")
    wl = synth.packed_wavefront()
    Kc, Vc, Q, o = _dev(wl)
    step = BlockDiffusionStep(Kc, Vc, Q, o, wl.bl, wl.sm_scale, p_max_dense=int(wl.o.max()))
    out = step.run().clone()
    out2 = step.run()
    torch.cuda.synchronize()
    ref, _ = orc.cache_attention_eq6(wl.Q, wl.Kc, wl.Vc, wl.o, wl.bl, wl.sm_scale)
    check_attention(out, ref, torch.bfloat16, label="packed_wavefront")
    assert torch.equal(out, out2), "a repeated step changed the output"
    ref_k = orc.kv_scatter(bits(wl.Kc)[None], bits(wl.Kc)[None], wl.o, wl.t, wl.q)[0]
    ref_v = orc.kv_scatter(bits(wl.Vc)[None], bits(wl.Vc)[None], wl.o, wl.t, wl.q)[0]
    assert np.array_equal(bits(Kc), ref_k) and np.array_equal(bits(Vc), ref_v)


def _sparse_block(bd, wl, label):
    """Select + gather once per block, then T denoising-step attentions over
    the pool plus the step's in-block KV."""
    note(f"config {label}: select")
    Kc, Vc = wl.Kc.cuda(), wl.Vc.cuda()
    B, Hkv, d = wl.B, wl.Hkv, wl.d
    k_max, s_max = wl.k_max, wl.s_max
    scores = torch.empty((B, Hkv, s_max), dtype=torch.float32, device="cuda")
    idx = bd.select(wl.Qsel.cuda(), Kc, wl.s_len.cuda(), s_max, wl.k_sel.cuda(), k_max,
                    wl.sm_scale, score_out=scores)
    pool_k = torch.zeros((B, k_max, Hkv, d), dtype=torch.bfloat16, device="cuda")
    pool_v = torch.zeros_like(pool_k)
    bd.gather(Kc, Vc, idx, wl.k_sel.cuda(), pool_k, pool_v)
    torch.cuda.synchronize()
    sc = scores.cpu().double().numpy()
    q_rep = orc.rep_query(wl.Qsel, "mean")
    ref_sc, _, _ = orc.selection_scores(q_rep, wl.Kc, wl.s_len, wl.sm_scale)
    check_scores(sc, ref_sc, wl.s_len, label)
    idx_ref = orc.topk_select(sc, wl.s_len, wl.k_sel, k_max)
    assert np.array_equal(idx.cpu().numpy(), idx_ref), f"{label}: indices differ"
    for (b, h), pos in wl.planted.items():
        assert set(pos.tolist()) <= set(idx_ref[b, h].tolist()), f"{label}: planted key missed"
    zeros = np.zeros((B, k_max, Hkv, d), np.int16)
    ref_pk = orc.gather(bits(wl.Kc), idx_ref, wl.k_sel, zeros)
    ref_pv = orc.gather(bits(wl.Vc), idx_ref, wl.k_sel, zeros)
    assert np.array_equal(bits(pool_k), ref_pk) and np.array_equal(bits(pool_v), ref_pv)
    pk64 = torch.from_numpy(ref_pk).view(torch.bfloat16)
    pv64 = torch.from_numpy(ref_pv).view(torch.bfloat16)
    for st in range(wl.T):
        note(f"config {label}: denoising step {st}")
        Qs = wl.extra["step_q"][st]
        wk, wv = wl.extra["step_kv"][st]
        out = bd.attn_packed(Qs.cuda(), pool_k, pool_v, wl.k_sel.cuda(), k_max, wk.cuda(),
                             wv.cuda(), wl.bl, wl.sm_scale)
        torch.cuda.synchronize()
        ref, _ = orc.block_attention(Qs, pk64, pv64, wl.k_sel, wk, wv, wl.bl, wl.sm_scale)
        check_attention(out, ref, torch.bfloat16, label=f"{label} step {st}")


def test_sparse_32k_config(bd):
    _sparse_block(bd, synth.sparse_32k(), "sparse_32k")


def test_sparse_128k_config(bd):
    _sparse_block(bd, synth.sparse_128k(), "sparse_128k")


def test_serving_mix_config(bd):
    """64 rows, log-uniform prefixes 1K-16K, W = 4; rows over 8K are sparse
    (5 % budget, representative query = mean of the row's window queries)."""
    from sparse_kv_cache_bd_amd.pipeline import BlockDiffusionStep
    note("config serving_mix: generate")
    wl = synth.serving_mix()
    Kc, Vc, Q, o = _dev(wl)
    step = BlockDiffusionStep(Kc, Vc, Q, o, wl.bl, wl.sm_scale, sparse_rows=wl.sparse_rows,
                              dense_rows=wl.dense_rows, s_len=wl.s_len, k_sel=wl.k_sel,
                              p_max_dense=int(wl.o[wl.dense_rows.long()].max()),
                              k_max=wl.k_max, s_max=wl.s_max)
    note("config serving_mix: step")
    out = step.run()
    torch.cuda.synchronize()
    sparse = wl.sparse_rows.tolist()
    dense = wl.dense_rows.tolist()
    assert len(sparse) > 0 and len(dense) > 0
    # selection of the sparse rows
    sc = step.scores.cpu().double().numpy()
    q_rep = orc.rep_query(wl.Q, "mean")
    ref_sc, _, _ = orc.selection_scores(q_rep, wl.Kc, wl.s_len, wl.sm_scale)
    check_scores(sc, ref_sc, wl.s_len, "serving_mix")
    idx_ref = orc.topk_select(sc, wl.s_len, wl.k_sel, wl.k_max)
    assert np.array_equal(step.idx.cpu().numpy(), idx_ref)
    zeros = np.zeros((wl.B, wl.k_max, wl.Hkv, wl.d), np.int16)
    ref_pk = orc.gather(bits(wl.Kc), idx_ref, wl.k_sel, zeros)
    ref_pv = orc.gather(bits(wl.Vc), idx_ref, wl.k_sel, zeros)
    gk, gv = bits(step.pool_k), bits(step.pool_v)
    for b in sparse:
        kb = int(wl.k_sel[b])
        assert np.array_equal(gk[b, :kb], ref_pk[b, :kb]) and np.array_equal(gv[b, :kb], ref_pv[b, :kb])
    # attention: every sparse row; dense rows sampled (longest, shortest, four more)
    pk = torch.from_numpy(ref_pk).view(torch.bfloat16)
    pv = torch.from_numpy(ref_pv).view(torch.bfloat16)
    t = wl.t
    ref_s, _ = orc.block_attention(wl.Q, pk, pv, wl.k_sel, wl.Kc[:, t:], wl.Vc[:, t:], wl.bl,
                                   wl.sm_scale, rows=sparse)
    check_attention(out, ref_s, torch.bfloat16, rows=sparse, label="serving_mix sparse")
    od = [(int(wl.o[b]), b) for b in dense]
    od.sort()
    sample = sorted({od[0][1], od[-1][1]} | {od[i][1] for i in np.linspace(1, len(od) - 2, 4).astype(int)})
    ref_d, _ = orc.block_attention(wl.Q, wl.Kc, wl.Vc, wl.o, wl.Kc[:, t:], wl.Vc[:, t:], wl.bl,
                                   wl.sm_scale, rows=sample)
    check_attention(out, ref_d, torch.bfloat16, rows=sample, label="serving_mix dense")
    # scatter: every row's target range holds the window; a sampled band of
    # untouched positions is unchanged
    Kafter = Kc.cpu()
    ka, k0 = bits(Kafter), bits(wl.Kc)
    for b in range(wl.B):
        ob = int(wl.o[b])
        assert np.array_equal(ka[b, ob:ob + wl.q], k0[b, t:t + wl.q])
        assert np.array_equal(ka[b, :ob:97], k0[b, :ob:97])
        assert np.array_equal(ka[b, t:], k0[b, t:])
