"""GPU check of the dual-stream sparse-block schedule (HERALD Sec. IV-B2):
block n+1's selection and gather on a second stream, overlapped with block
n's denoising attentions on the main stream, double-buffered pools.  The
overlapped run must give bit-identical pools and outputs to the same calls
issued in order on one stream, and the last step's output must match the
float64 oracle's attention over the gathered pool.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import bits, check_attention, note
from oracle import bd_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


@pytest.mark.parametrize("T,n_blocks", [(4, 3), (1, 2), (2, 4)])
def test_overlapped_equals_sequential(bd, T, n_blocks):
    from sparse_kv_cache_bd_amd.pipeline import SparseBlockPipeline
    note(f"pipeline T={T} blocks={n_blocks}")
    wl = synth.sparse_32k(B=2, S=8192, T=T)
    Kc, Vc = wl.Kc.cuda(), wl.Vc.cuda()
    steps_q = [x.cuda() for x in wl.extra["step_q"]]
    steps_kv = [(a.cuda(), b.cuda()) for a, b in wl.extra["step_kv"]]

    def make():
        return SparseBlockPipeline(Kc, Vc, wl.Qsel.cuda(), wl.s_len.cuda(), wl.k_sel.cuda(),
                                   wl.s_max, wl.k_max, wl.sm_scale, wl.bl, steps_q, steps_kv)
    seq, ovl = make(), make()
    out_s = seq.run_sequential(n_blocks).clone()
    out_o = ovl.run_overlapped(n_blocks).clone()
    out_o2 = ovl.run_overlapped(n_blocks).clone()
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_o) and torch.equal(out_o, out_o2)
    for slot in range(2 if n_blocks > 1 else 1):
        for a, b in zip(seq.pools[slot], ovl.pools[slot]):
            assert torch.equal(a, b)
    assert torch.equal(seq.idx, ovl.idx)
    # the last step over the last block's pool against the oracle
    last = (n_blocks - 1) % 2
    kb = wl.k_sel.numpy()
    idx = seq.idx.cpu().numpy()
    zeros = np.zeros((wl.B, wl.k_max, wl.Hkv, wl.d), np.int16)
    pk_ref = orc.gather(bits(wl.Kc), idx, kb, zeros)
    assert np.array_equal(bits(seq.pools[last][0])[:, :int(kb.max())], pk_ref[:, :int(kb.max())])
    wk, wv = wl.extra["step_kv"][T - 1]
    ref, _ = orc.block_attention(wl.extra["step_q"][T - 1], seq.pools[last][0].cpu(),
                                 seq.pools[last][1].cpu(), wl.k_sel, wk, wv, wl.bl, wl.sm_scale)
    check_attention(out_s, ref, torch.bfloat16, label="pipeline")


def test_denoising_steps_in_a_hip_graph(bd):
    """The T denoising attentions over one pool captured in a HIP graph: every
    replay (with eager work and synchronisations between replays) gives the
    eager outputs bit for bit."""
    note("denoising steps in a HIP graph")
    wl = synth.sparse_32k(B=2, S=8192, T=3)
    Kc, Vc = wl.Kc.cuda(), wl.Vc.cuda()
    idx = bd.select(wl.Qsel.cuda(), Kc, wl.s_len.cuda(), wl.s_max, wl.k_sel.cuda(), wl.k_max,
                    wl.sm_scale)
    pk = torch.zeros((wl.B, wl.k_max, wl.Hkv, wl.d), dtype=torch.bfloat16, device="cuda")
    pv = torch.zeros_like(pk)
    k_sel = wl.k_sel.cuda()
    bd.gather(Kc, Vc, idx, k_sel, pk, pv)
    steps_q = [x.cuda() for x in wl.extra["step_q"]]
    steps_kv = [(a.cuda(), b.cuda()) for a, b in wl.extra["step_kv"]]
    outs = [torch.empty_like(steps_q[0]) for _ in range(wl.T)]
    ws = bd.workspace(bd.attn_workspace_size(torch.bfloat16, wl.B, wl.Hq, wl.Hkv, wl.d, wl.q,
                                             wl.B, wl.k_max), "cuda")

    def steps():
        for st in range(wl.T):
            wk, wv = steps_kv[st]
            bd.attn_packed(steps_q[st], pk, pv, k_sel, wl.k_max, wk, wv, wl.bl, wl.sm_scale,
                           out=outs[st], ws=ws)
    steps()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps()
    for rep in range(3):
        for o in outs:
            o.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for st in range(wl.T):
            assert torch.equal(outs[st], want[st]), f"replay {rep}, step {st}"
        bd.select(wl.Qsel.cuda(), Kc, wl.s_len.cuda(), wl.s_max, k_sel, wl.k_max, wl.sm_scale)


def test_budget_above_prefix(bd):
    """A row whose budget exceeds its prefix (k_b > S_b) keeps all S_b
    positions; its pool holds S_b entries and its attention covers exactly
    those, never the pool slots past them (which hold stale values)."""
    from sparse_kv_cache_bd_amd.pipeline import BlockDiffusionStep, SparseBlockPipeline
    note("pipeline: budget above the prefix")
    wl = synth.serving_mix(seed=3, B=3, p_lo=200, p_hi=1200, W=2, sparse_above=100)
    k_sel = wl.k_sel.clone()
    k_sel[0] = int(wl.s_len[0]) + 77          # more than the row's prefix
    k_max = int(k_sel.max())
    Kc, Vc, Q, o = wl.Kc.cuda(), wl.Vc.cuda(), wl.Q.cuda(), wl.o.cuda()
    step = BlockDiffusionStep(Kc, Vc, Q, o, wl.bl, wl.sm_scale, sparse_rows=wl.sparse_rows,
                              dense_rows=wl.dense_rows, s_len=wl.s_len, k_sel=k_sel,
                              p_max_dense=int(wl.o.max()), k_max=k_max, s_max=wl.s_max)
    step.pool_k.fill_(float("nan"))          # stale pool content must never be read
    step.pool_v.fill_(float("nan"))
    step.select()
    step.gather()
    step.attn_sparse()
    torch.cuda.synchronize()
    k_eff = np.minimum(k_sel.numpy(), wl.s_len.numpy())
    idx = orc.topk_select(step.scores.cpu().double().numpy(), wl.s_len, k_sel, k_max)
    assert np.array_equal(step.idx.cpu().numpy(), idx)
    assert (idx[0, :, :int(wl.s_len[0])] == np.arange(int(wl.s_len[0]))).all()
    zeros = np.zeros((wl.B, k_max, wl.Hkv, wl.d))
    pk = orc.gather(wl.Kc.double().numpy(), idx, k_eff, zeros)
    pv = orc.gather(wl.Vc.double().numpy(), idx, k_eff, zeros)
    t = wl.t
    rows = wl.sparse_rows.tolist()
    ref, _ = orc.block_attention(wl.Q, pk, pv, k_eff, wl.Kc[:, t:], wl.Vc[:, t:], wl.bl,
                                 wl.sm_scale, rows=rows)
    check_attention(step.out, ref, torch.bfloat16, rows=rows, label="budget above prefix")
    # the dual-stream pipeline takes the same pool length
    sel = torch.tensor(rows, dtype=torch.long)
    pipe = SparseBlockPipeline(Kc[sel], Vc[sel], Q[sel], wl.s_len[sel].cuda(), k_sel[sel].cuda(),
                               wl.s_max, k_max, wl.sm_scale, wl.bl, [Q[sel]],
                               [(Kc[sel][:, t:], Vc[sel][:, t:])])
    for pk_, pv_ in pipe.pools:
        pk_.fill_(float("nan"))
        pv_.fill_(float("nan"))
    out = pipe.run_sequential(1)
    torch.cuda.synchronize()
    check_attention(out, ref[sel.numpy()], torch.bfloat16, label="budget above prefix, pipeline")
