"""Benchmark of the block-diffusion hot path on one MI355X.

One step = one pass of every operation of the path over one batch of the
64-row serving mix (log-uniform prefixes 1K-16K, W = 4 windows of 32-token
blocks, 32/8 heads, d = 128, bf16): selection + gather for the rows whose
prefix exceeds 8K (5 % budget), W-shaped attention of the dense rows over
their own cache and of the sparse rows over their pools (one launch for
both), and the KV write-back scatter of every row.  Inputs are resident in
HBM before the timed region.

Before the ``--warmup`` steps an untimed settle phase repeats the step for
a fixed wall time (``--settle-ms``, default 400 ms; reported as
``settle_ms`` / ``settle_steps``): the first few dozen steps of a fresh
process run up to 15 % slower than steady state (the attention launch
448-580 us against 404 us), so a short warm-up alone would time the ramp.
The timed region holds exactly ``--steps`` steps with no event between
operations; a second pass over the same number of steps records an event
after every operation for ``breakdown`` (those events add about 8 us per
step).

Prints one JSON line.  ``value`` is the whole-step throughput in attention
TFLOP/s: the algorithmic attention FLOPs of the step (4*d per visible
(query, key) pair per query head) divided by the step time, select, gather
and scatter included.  ``breakdown`` gives each operation's own rate
(TFLOP/s or GB/s of algorithmic bytes) and fraction of the MI355X peak.
``roofline`` reports the dominant kernel (the attention launch over all
rows), timed with HIP events on the stream it runs on; ``attn_dense`` and
``attn_sparse`` in ``breakdown`` time the two row kinds as separate
launches for reference.  ``cpu_baseline`` times the float64
oracle on a bounded sample of the same step on the host cores.  ``configs``
adds the other synthetic workloads (tiny fp32 block, packed wavefronts,
sparse 32K and 128K prefixes) operation by operation.

``--only OP`` times one operation of the step (for counter runs) and
``--copy-probe MB`` runs a plain device copy of known size, whose
FETCH_SIZE / WRITE_SIZE counters scale the attention's.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "block-diffusion attn TFLOP/s + select GB/s, as % of MI355X roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_mfma_serving_mix_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "sparse_kv_cache_bd_amd", "csrc", "bd_attn.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def window_keys(i, q, bl, mode="block_causal"):
    """Window keys query i sees under each window mask."""
    lim = min(q, (i // bl + 1) * bl)
    if mode == "block_causal":
        return lim
    own = lim - (i // bl) * bl
    return own if (mode == "isolated" or i < bl) else own + bl


def attention_flops(p_len, rows, q, bl, Hq, d, mode="block_causal"):
    """4*d FLOPs per visible (query, key) pair per query head."""
    win = sum(window_keys(i, q, bl, mode) for i in range(q))
    return sum(4 * d * Hq * (q * int(p_len[b]) + win) for b in rows)


def step_work(wl):
    """Algorithmic FLOPs / bytes of one step, per operation."""
    q, bl, Hq, Hkv, d = wl.q, wl.bl, wl.Hq, wl.Hkv, wl.d
    es = 2
    dense = wl.dense_rows.tolist()
    sparse = wl.sparse_rows.tolist()
    tok = Hkv * d * es                      # bytes of one (pos) row of K or V
    w = {}
    w["attn_dense_flop"] = attention_flops(wl.o, dense, q, bl, Hq, d)
    w["attn_sparse_flop"] = attention_flops(wl.k_sel, sparse, q, bl, Hq, d)
    w["select_bytes"] = sum(int(wl.s_len[b]) * tok for b in sparse) + len(sparse) * Hkv * wl.k_max * 4
    w["gather_bytes"] = sum(int(wl.k_sel[b]) * tok * 2 * 2 for b in sparse)
    w["scatter_bytes"] = wl.B * q * tok * 2 * 2
    # bytes the attention must move at least once: Q, O, prefix (cache or
    # pool) + window K/V
    w["attn_dense_bytes"] = sum(q * Hq * d * es * 2 + (int(wl.o[b]) + q) * tok * 2 for b in dense)
    w["attn_sparse_bytes"] = sum(q * Hq * d * es * 2 + (int(wl.k_sel[b]) + q) * tok * 2 for b in sparse)
    return w


def traffic_for_attention():
    """HBM bytes per attention launch (all rows) from the committed rocprofv3
    counter summary, or None when the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(ATTN_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if rec.get("source_sha256") != sha:
            return None
        return rec.get("bytes_per_launch")
    except (OSError, ValueError):
        return None


def cpu_baseline(wl, budget_s: float = 25.0):
    """The float64 oracle timed on the host cores over a bounded sample of
    the same step: whole rows (selection + gather + attention for sparse
    rows, attention for dense rows, then the scatter), alternating dense and
    sparse rows from the shortest up until about ``budget_s`` seconds."""
    import numpy as np
    import torch
    from oracle import bd_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    dense = sorted(wl.dense_rows.tolist(), key=lambda b: int(wl.o[b]))
    sparse = sorted(wl.sparse_rows.tolist(), key=lambda b: int(wl.o[b]))
    order = []
    for i in range(max(len(dense), len(sparse))):
        if i < len(dense):
            order.append(("dense", dense[i]))
        if i < len(sparse):
            order.append(("sparse", sparse[i]))
    t = wl.t
    flops = 0
    done = []
    t0 = time.perf_counter()
    for kind, b in order:
        rows = [b]
        if kind == "dense":
            orc.block_attention(wl.Q[b:b + 1], wl.Kc[b:b + 1], wl.Vc[b:b + 1], wl.o[b:b + 1],
                                wl.Kc[b:b + 1, t:], wl.Vc[b:b + 1, t:], wl.bl, wl.sm_scale)
            flops += attention_flops(wl.o, rows, wl.q, wl.bl, wl.Hq, wl.d)
        else:
            qr = orc.rep_query(wl.Q[b:b + 1], "mean")
            sh, _, _ = orc.selection_scores(qr, wl.Kc[b:b + 1], wl.s_len[b:b + 1], wl.sm_scale)
            idx = orc.topk_select(sh, wl.s_len[b:b + 1], wl.k_sel[b:b + 1], int(wl.k_sel[b]))
            kb = int(wl.k_sel[b])
            z = np.zeros((1, kb, wl.Hkv, wl.d))
            pk = orc.gather(wl.Kc[b:b + 1].double().numpy(), idx, wl.k_sel[b:b + 1], z)
            pv = orc.gather(wl.Vc[b:b + 1].double().numpy(), idx, wl.k_sel[b:b + 1], z)
            orc.block_attention(wl.Q[b:b + 1], pk, pv, wl.k_sel[b:b + 1], wl.Kc[b:b + 1, t:],
                                wl.Vc[b:b + 1, t:], wl.bl, wl.sm_scale)
            flops += attention_flops(wl.k_sel, rows, wl.q, wl.bl, wl.Hq, wl.d)
        kv = wl.Kc[b:b + 1].view(torch.int16).numpy()[None]
        orc.kv_scatter(kv, kv, wl.o[b:b + 1], t, wl.q)
        done.append(f"{kind}:{b}(P={int(wl.o[b])})")
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"all {wl.B} rows of the same step" if len(done) == wl.B else
                       f"{len(done)} of {wl.B} rows of the same step, shortest first") +
                      f", whole rows (dense: attention; sparse: select+gather+attention; all: "
                      f"scatter): {', '.join(done)}; {el:.1f} s float64 NumPy",
            "seconds": round(el, 2)}


def time_calls(fn, reps: int, warmup: int = 2, settle_ms: float = 100.0) -> float:
    """Average milliseconds per call of ``fn`` (HIP events on the current
    stream, which is the stream the library launches on).  Before the timed
    calls, ``fn`` runs untimed for at least ``settle_ms`` of wall time (the
    GPU's clocks settle at the load; a first call after an idle gap runs up
    to 20 % slower), then ``warmup`` more times.  A spin kernel ahead of the
    first event gives the host time to queue every call, so short calls are
    timed back to back on the GPU, not at the host's launch rate."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda._sleep(400_000)   # about 0.2 ms: the host gets ahead and stays ahead
    ev[0].record()
    for i in range(reps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return sum(ev[i].elapsed_time(ev[i + 1]) for i in range(reps)) / reps


def _rate(num, ms, scale):
    return round(num / (ms * 1e-3) / scale, 2)


FLUSH_BYTES = 512 << 20   # larger than the MALL (256 MB) plus every L2


def time_cold(fn, flush, reps: int):
    """Milliseconds per call of ``fn`` with L2 and MALL flushed before each
    call, outside the event pair: (median, p10, p90).  The flush reads a
    512 MB buffer (an int64 sum), so the caches then hold clean lines; a
    flush by writing would leave up to 256 MB of dirty lines whose write-back
    the timed call would pay for."""
    import torch
    ts = []
    for i in range(reps + 1):
        flush.view(torch.int64).sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        if i > 0:   # the first call is a warm-up
            ts.append(e0.elapsed_time(e1))
    ts.sort()
    q = lambda f: ts[min(len(ts) - 1, int(f * (len(ts) - 1) + 0.5))]
    return q(0.5), q(0.1), q(0.9)


def attainable_tflops(flop, nbytes, peak_tflops):
    """min(MFMA peak, intensity x HBM peak)."""
    return min(peak_tflops, flop / nbytes * PEAK_HBM_GBS / 1e3)


def select_multi_sweep(bd, wl, Kc, s_len, k_sel, sel_bytes, ms_rep, dev, reps):
    """Exact multi-query selection (every one of nq block queries ranks the
    prefix) against the query count, as HERALD's Fig. 8 sweeps it: time per
    call, K bytes read once over the call time (the kernels read K twice),
    logit FLOPs (2*d per (query, query head, token)) and throughput relative
    to nq = 32.  ``rep_mean_us`` is bd_select with the mean query."""
    import torch
    B, Hq, Hkv, d, k_max, s_max = wl.B, wl.Hq, wl.Hkv, wl.d, wl.k_max, wl.s_max
    idx = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=dev)
    tokens = sum(int(wl.s_len[b]) for b in range(B))
    res = {"rep_mean_us": round(ms_rep * 1e3, 2)}
    for nq in (1, 2, 4, 8, 16, 32):
        Qn = wl.Qsel[:, :nq].contiguous().to(dev)
        ws = bd.workspace(bd.select_multi_workspace_size(B, Hq, Hkv, d, nq, s_max, k_max), dev)
        ms = time_calls(lambda: bd.select_multi(Qn, Kc, s_len, s_max, k_sel, k_max, wl.sm_scale,
                                                idx_out=idx, ws=ws), reps)
        res[str(nq)] = {"us": round(ms * 1e3, 2), "GB/s": _rate(sel_bytes, ms, 1e9),
                        "frac_hbm_once": round(sel_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "frac_hbm_two_passes": round(2 * sel_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "logit_TFLOP/s": _rate(2 * d * nq * Hq * tokens, ms, 1e12)}
        del ws
    base = res["32"]["us"]
    for nq in (1, 2, 4, 8, 16, 32):
        res[str(nq)]["speedup_vs_32"] = round(base / res[str(nq)]["us"], 3)
    return res


def hbm_reference(dev, reps: int = 20) -> dict:
    """Streaming rates of torch's own device kernels on 1 GiB fp32 buffers:
    copy (read + write), sum (read) and fill (write), as the practical HBM
    reference next to the 8 TB/s peak."""
    import torch
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    nb = n * 4
    out = {"bytes": nb,
           "copy_TB/s": round(2 * nb / (time_calls(lambda: b.copy_(a), reps) * 1e-3) / 1e12, 2),
           "read_TB/s": round(nb / (time_calls(lambda: a.sum(), reps) * 1e-3) / 1e12, 2),
           "write_TB/s": round(nb / (time_calls(lambda: b.fill_(1.0), reps) * 1e-3) / 1e12, 2)}
    del a, b
    torch.cuda.empty_cache()
    return out


def bench_producer(bd, dev, reps):
    """Flash-dLLM's fused cache producer (QKV projection + RoPE + cache write)
    at the serving-mix shape: 64 rows x 128 window tokens, hidden 4096 (32
    query heads x 128), 32/8 heads; keys and values written at the window
    tail of a [64, 16640, 8, 128] cache.  Synthetic N(0,1) hidden states and
    N(0,1)/sqrt(4096) weights."""
    import torch
    B, q, Dm, Hq, Hkv, d, C = 64, 128, 4096, 32, 8, 128, 16640
    g = torch.Generator(device=dev).manual_seed(0)
    X = torch.randn((B, q, Dm), generator=g, device=dev).bfloat16()
    W = (torch.randn(((Hq + 2 * Hkv) * d, Dm), generator=g, device=dev) / math.sqrt(Dm)).bfloat16()
    Kc = torch.zeros((B, C, Hkv, d), dtype=torch.bfloat16, device=dev)
    Vc = torch.zeros_like(Kc)
    Qo = torch.empty((B, q, Hq, d), dtype=torch.bfloat16, device=dev)
    rope_pos = torch.randint(1024, 16384, (B,), generator=g, device=dev).to(torch.int32)
    dst = torch.full((B,), C - q, dtype=torch.int32, device=dev)
    ms = time_calls(lambda: bd.qkv_rope_write(X, W, rope_pos, Hq, Hkv, Qo, Kc, Vc, dst), reps)
    flop = 2 * B * q * Dm * (Hq + 2 * Hkv) * d
    nbytes = (B * q * Dm + (Hq + 2 * Hkv) * d * Dm + B * q * (Hq + 2 * Hkv) * d) * 2
    # the same work unfused, as the separate launches a framework issues:
    # the projection as one library GEMM (hipBLASLt through torch), RoPE of
    # the query and key heads as elementwise ops, then the copy of keys and
    # values into the cache tail
    t = C - q
    j = torch.arange(d // 2, device=dev, dtype=torch.float64)
    inv_freq = torch.pow(torch.tensor(10000.0, dtype=torch.float64, device=dev), -2.0 * j / d)
    pos = rope_pos.to(torch.float64)[:, None] + torch.arange(q, device=dev, dtype=torch.float64)[None, :]
    ang = pos[:, :, None] * inv_freq                          # [B, q, d/2]
    cos = torch.cos(ang).float()[:, :, None, :]
    sin = torch.sin(ang).float()[:, :, None, :]

    Wt = W.t().contiguous()      # the library GEMM takes a plain [Dm, N] operand

    def unfused():
        Y = torch.matmul(X.view(B * q, Dm), Wt).view(B, q, Hq + 2 * Hkv, d)
        qk = Y[:, :, :Hq + Hkv].float()
        x1, x2 = qk[..., :d // 2], qk[..., d // 2:]
        rot = torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1).bfloat16()
        Qo.copy_(rot[:, :, :Hq])
        Kc[:, t:].copy_(rot[:, :, Hq:])
        Vc[:, t:].copy_(Y[:, :, Hq + Hkv:])

    ms_unf = time_calls(unfused, reps)
    ms_gemm = time_calls(lambda: torch.matmul(X.view(B * q, Dm), Wt), reps)
    res = {"tokens": B * q, "hidden": Dm, "heads": [Hq, Hkv], "us": round(ms * 1e3, 2),
           "TFLOP/s": _rate(flop, ms, 1e12),
           "frac_mfma_peak": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "gflop": round(flop / 1e9, 1), "min_mb": round(nbytes / 1e6, 1),
           "unfused_us": round(ms_unf * 1e3, 2),
           "unfused_gemm_only_us": round(ms_gemm * 1e3, 2),
           "unfused_gemm_TFLOP/s": _rate(flop, ms_gemm, 1e12),
           "fused_speedup_vs_unfused": round(ms_unf / ms, 3)}
    del X, W, Wt, Kc, Vc, Qo
    torch.cuda.empty_cache()
    return res


def bench_block_table(bd, wl, Kc, Vc, Q, dense_pmax, ms_packed, reps, page=128):
    """Flash-dLLM's Scheduled Flash Attention on the serving mix's dense
    rows: each row's prefix cut into pages of ``page`` keys at shuffled slots
    of a paged store, one work item per row, dispatched in row order and
    longest first (the caller's choice), against bd_attn_packed over the
    same rows (contiguous cache, the library's own longest-first order)."""
    import torch
    rows = wl.dense_rows.long().to(Kc.device)
    P = wl.o.long().to(Kc.device)[rows]
    n_pg = (P + page - 1) // page
    total = int(n_pg.sum())
    row_of = torch.repeat_interleave(rows, n_pg)
    first = torch.cumsum(n_pg, 0) - n_pg
    j_of = torch.arange(total, device=Kc.device) - torch.repeat_interleave(first, n_pg)
    g = torch.Generator(device=Kc.device).manual_seed(0)
    slot = torch.randperm(total, generator=g, device=Kc.device)
    pos = (j_of[:, None] * page + torch.arange(page, device=Kc.device)[None, :]).clamp_(max=Kc.shape[1] - 1)
    KP = torch.empty((total, page, wl.Hkv, wl.d), dtype=Kc.dtype, device=Kc.device)
    VP = torch.empty_like(KP)
    KP[slot] = Kc[row_of[:, None], pos]
    VP[slot] = Vc[row_of[:, None], pos]
    table = slot.to(torch.int32)
    items = torch.stack([rows, torch.zeros_like(rows), torch.full_like(rows, wl.q), first, P], 1).to(torch.int32)
    longest = items[torch.argsort(P, descending=True, stable=True)].contiguous()
    wk, wv = Kc[:, wl.t:], Vc[:, wl.t:]
    out = torch.empty_like(Q)
    ws = bd.workspace(bd.attn_block_table_workspace_size(Q.dtype, wl.Hq, wl.Hkv, wl.d, wl.q,
                                                         len(items), dense_pmax), Q.device)
    res = {"rows": len(items), "page": page, "pages": total,
           "store_mb": round(2 * KP.numel() * 2 / 1e6, 1)}
    flop = attention_flops(wl.o, wl.dense_rows.tolist(), wl.q, wl.bl, wl.Hq, wl.d)
    for name, it in (("row_order", items.contiguous()), ("longest_first", longest)):
        ms = time_calls(lambda: bd.attn_block_table(Q, KP, VP, it, table, dense_pmax, wk, wv, wl.bl,
                                                    wl.sm_scale, out=out, ws=ws), reps)
        res[f"{name}_us"] = round(ms * 1e3, 2)
        res[f"{name}_TFLOP/s"] = _rate(flop, ms, 1e12)
    res["packed_contiguous_us"] = round(ms_packed * 1e3, 2)
    del KP, VP
    torch.cuda.empty_cache()
    return res


def bench_scatter_layers(bd, dev, reps):
    """FlowBlock's write-back, Eq. (7), applied to every layer: the scatter
    of one window per row for L layers in one call, on the packed-wavefront
    shape (8 rows, C = 4096, q = 64) and the serving-mix shape (64 rows,
    C = 16640, q = 128); 32/8 heads, d = 128, bf16.  Synthetic caches (the
    values are copied bit for bit, so uninitialised memory is timed)."""
    import torch
    res = {}
    for name, B, C, q, layers in (("packed_wavefront", 8, 4096, 64, (1, 8, 32)),
                                  ("serving_mix", 64, 16640, 128, (1, 8))):
        g = torch.Generator().manual_seed(1)
        o = (torch.randint(16, (C - 2 * q) // 32, (B,), generator=g) * 32).to(torch.int32).to(dev)
        for L in layers:
            Kc = torch.empty((L, B, C, 8, 128), dtype=torch.bfloat16, device=dev)
            Vc = torch.empty_like(Kc)
            ms = time_calls(lambda: bd.kv_scatter(Kc, Vc, Kc, Vc, o, C - q, q), reps)
            nbytes = L * B * q * 8 * 128 * 2 * 2 * 2
            res[f"{name}_L{L}"] = {"us": round(ms * 1e3, 2), "GB/s": _rate(nbytes, ms, 1e9),
                                   "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                   "mb": round(nbytes / 1e6, 1)}
            del Kc, Vc
            torch.cuda.empty_cache()
    return res


def bench_configs(dev, reps: int = 10):
    """The other synthetic workloads, each in the launch configuration its
    parity test checks: per-operation times and rates, warm (back-to-back
    calls, mean) and cold (L2 and MALL flushed before every call; median,
    p10, p90 in ``*_cold_us``)."""
    import torch
    import synth
    from sparse_kv_cache_bd_amd import bdattn as bd
    from sparse_kv_cache_bd_amd.pipeline import BlockDiffusionStep, SparseBlockPipeline
    out = {}
    flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    cold_reps = 20

    def cold(fn):
        med, p10, p90 = time_cold(fn, flush, cold_reps)
        return med, [round(med * 1e3, 2), round(p10 * 1e3, 2), round(p90 * 1e3, 2)]

    def kv_bytes(wl):
        return wl.Hkv * wl.d * (2 if wl.dtype == "bf16" else 4)

    for name in ("tiny_dense", "packed_wavefront"):
        log(f"config {name}")
        wl = getattr(synth, name)()
        Kc, Vc, Q, o = (x.to(dev) for x in (wl.Kc, wl.Vc, wl.Q, wl.o))
        step = BlockDiffusionStep(Kc, Vc, Q, o, wl.bl, wl.sm_scale, p_max_dense=int(wl.o.max()))
        ms_a = time_calls(step.attn_dense, reps)
        ms_s = time_calls(step.scatter, reps)
        # the other window masks on the same rows (HERALD's isolated
        # draft/denoise groups; Flash-dLLM's verify views)
        modes = {}
        if wl.W > 1:
            for mode in ("isolated", "shared_first"):
                out_m = torch.empty_like(Q)
                fm = lambda: bd.attn_packed(Q, Kc, Vc, o, int(wl.o.max()), step.wk, step.wv, wl.bl,
                                            wl.sm_scale, out=out_m, ws=step.ws_dense, mask_mode=mode)
                ms_m = time_calls(fm, reps)
                fl = attention_flops(wl.o, range(wl.B), wl.q, wl.bl, wl.Hq, wl.d, mode)
                modes[mode] = {"us": round(ms_m * 1e3, 2), "TFLOP/s": _rate(fl, ms_m, 1e12)}
        ms_ac, q_ac = cold(step.attn_dense)
        ms_sc, q_sc = cold(step.scatter)
        flop = attention_flops(wl.o, range(wl.B), wl.q, wl.bl, wl.Hq, wl.d)
        es = 2 if wl.dtype == "bf16" else 4
        abytes = sum(wl.q * wl.Hq * wl.d * es * 2 + (int(wl.o[b]) + wl.q) * kv_bytes(wl) * 2
                     for b in range(wl.B))
        sbytes = wl.B * wl.q * kv_bytes(wl) * 2 * 2
        unit_peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else 157.3
        att = attainable_tflops(flop, abytes, unit_peak)
        out[name] = {"dtype": wl.dtype, "rows": wl.B, "q": wl.q,
                     "attn_us": round(ms_a * 1e3, 2), "attn_TFLOP/s": _rate(flop, ms_a, 1e12),
                     "attn_frac_peak": round(flop / (ms_a * 1e-3) / 1e12 / unit_peak, 4),
                     "attn_cold_us": q_ac,
                     "attn_cold_frac_attainable": round(flop / (ms_ac * 1e-3) / 1e12 / att, 4),
                     "attainable_TFLOP/s": round(att, 1),
                     "scatter_us": round(ms_s * 1e3, 2), "scatter_GB/s": _rate(sbytes, ms_s, 1e9),
                     "scatter_cold_us": q_sc, "scatter_cold_GB/s": _rate(sbytes, ms_sc, 1e9)}
        if modes:
            out[name]["attn_other_masks"] = modes
        del step, Kc, Vc, Q, o

    for name in ("sparse_32k", "sparse_128k"):
        log(f"config {name}")
        wl = getattr(synth, name)()
        Kc, Vc = wl.Kc.to(dev), wl.Vc.to(dev)
        Qsel = wl.Qsel.to(dev)
        s_len, k_sel = wl.s_len.to(dev), wl.k_sel.to(dev)
        B, Hkv, d, k_max, s_max = wl.B, wl.Hkv, wl.d, wl.k_max, wl.s_max
        idx = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=dev)
        ws = bd.workspace(bd.select_workspace_size(B, wl.Hq, Hkv, d, s_max, k_max), dev)
        pool_k = torch.zeros((B, k_max, Hkv, d), dtype=Kc.dtype, device=dev)
        pool_v = torch.zeros_like(pool_k)
        f_sel = lambda: bd.select(Qsel, Kc, s_len, s_max, k_sel, k_max, wl.sm_scale, idx_out=idx, ws=ws)
        f_gat = lambda: bd.gather(Kc, Vc, idx, k_sel, pool_k, pool_v)
        ms_sel = time_calls(f_sel, reps)
        # the same selection plus the representative query's attention
        # output over the prefix (V read once more)
        o_rep = torch.empty((B, wl.Hq, d), dtype=Kc.dtype, device=dev)
        ws_o = bd.workspace(bd.select_attn_workspace_size(B, wl.Hq, Hkv, d, s_max, k_max), dev)
        ms_sela = time_calls(lambda: bd.select_attn(Qsel, Kc, Vc, s_len, s_max, k_sel, k_max, wl.sm_scale,
                                                    idx_out=idx, o_rep=o_rep, ws=ws_o), reps)
        del ws_o
        ms_gat = time_calls(f_gat, reps)
        ms_selc, q_selc = cold(f_sel)
        ms_gatc, q_gatc = cold(f_gat)
        steps_q = [x.to(dev) for x in wl.extra["step_q"]]
        steps_kv = [(a.to(dev), b.to(dev)) for a, b in wl.extra["step_kv"]]
        outb = torch.empty_like(steps_q[0])
        ws_a = bd.workspace(bd.attn_workspace_size(Qsel.dtype, B, wl.Hq, Hkv, d, wl.q, B, k_max), dev)

        def steps():
            for st in range(wl.T):
                wk, wv = steps_kv[st]
                bd.attn_packed(steps_q[st], pool_k, pool_v, k_sel, k_max, wk, wv, wl.bl,
                               wl.sm_scale, out=outb, ws=ws_a)
        ms_att = time_calls(steps, max(2, reps // 2))
        # the same T steps captured once in a HIP graph and replayed (the
        # step kernels are short: launch gaps are a visible share)
        graph = torch.cuda.CUDAGraph()
        steps()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            steps()
        graph.replay()
        torch.cuda.synchronize()
        ms_att_graph = time_calls(graph.replay, max(2, reps // 2))
        del graph
        wk0, wv0 = steps_kv[0]
        ms_attc, q_attc = cold(lambda: bd.attn_packed(steps_q[0], pool_k, pool_v, k_sel, k_max, wk0, wv0,
                                                      wl.bl, wl.sm_scale, out=outb, ws=ws_a))
        # HERALD's dual-stream schedule: block n+1's select + gather on a second
        # stream under block n's denoising steps, double-buffered pools
        pipe = SparseBlockPipeline(Kc, Vc, Qsel, s_len, k_sel, s_max, k_max, wl.sm_scale, wl.bl,
                                   steps_q, steps_kv)
        nb = 4
        ms_pseq = time_calls(lambda: pipe.run_sequential(nb), max(2, reps // 2)) / nb
        ms_povl = time_calls(lambda: pipe.run_overlapped(nb), max(2, reps // 2)) / nb
        del pipe
        sel_bytes = sum(int(wl.s_len[b]) for b in range(B)) * kv_bytes(wl) + B * Hkv * k_max * 4
        gat_bytes = sum(int(wl.k_sel[b]) for b in range(B)) * kv_bytes(wl) * 2 * 2
        flop1 = attention_flops(wl.k_sel, range(B), wl.q, wl.bl, wl.Hq, wl.d)
        flop = wl.T * flop1
        abytes1 = sum(wl.q * wl.Hq * wl.d * 2 * 2 + (int(wl.k_sel[b]) + wl.q) * kv_bytes(wl) * 2
                      for b in range(B))
        att = attainable_tflops(flop1, abytes1, PEAK_BF16_TFLOPS)
        sweep = None
        if name == "sparse_32k":
            sweep = select_multi_sweep(bd, wl, Kc, s_len, k_sel, sel_bytes, ms_sel, dev, reps)
        out[name] = {"rows": B, "prefix": s_max, "k": k_max, "T": wl.T,
                     "select_us": round(ms_sel * 1e3, 2), "select_GB/s": _rate(sel_bytes, ms_sel, 1e9),
                     "select_frac_hbm": round(sel_bytes / (ms_sel * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "select_cold_us": q_selc, "select_cold_GB/s": _rate(sel_bytes, ms_selc, 1e9),
                     "select_cold_frac_hbm": round(sel_bytes / (ms_selc * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "select_attn": {"us": round(ms_sela * 1e3, 2),
                                     "GB/s": _rate(sel_bytes + sum(int(wl.s_len[b]) for b in range(B))
                                                   * kv_bytes(wl), ms_sela, 1e9),
                                     "output_pass_us": round((ms_sela - ms_sel) * 1e3, 2)},
                     "gather_us": round(ms_gat * 1e3, 2), "gather_GB/s": _rate(gat_bytes, ms_gat, 1e9),
                     "gather_cold_us": q_gatc, "gather_cold_GB/s": _rate(gat_bytes, ms_gatc, 1e9),
                     "attn_us_per_step": round(ms_att * 1e3 / wl.T, 2),
                     "attn_us_per_step_graph": round(ms_att_graph * 1e3 / wl.T, 2),
                     "attn_TFLOP/s": _rate(flop, ms_att, 1e12),
                     "attn_cold_us_per_step": q_attc,
                     "attn_cold_frac_attainable": round(flop1 / (ms_attc * 1e-3) / 1e12 / att, 4),
                     "attainable_TFLOP/s": round(att, 1),
                     "block_us": round((ms_sel + ms_gat + ms_att) * 1e3, 2),
                     "pipeline": {"blocks": nb, "block_us_sequential": round(ms_pseq * 1e3, 2),
                                  "block_us_overlapped": round(ms_povl * 1e3, 2),
                                  "speedup": round(ms_pseq / ms_povl, 3)}}
        if sweep:
            out[name]["select_multi_sweep"] = sweep
        del Kc, Vc, pool_k, pool_v, ws, ws_a
        torch.cuda.empty_cache()
    out["producer_serving_mix"] = bench_producer(bd, dev, reps)
    out["scatter_layers"] = bench_scatter_layers(bd, dev, reps)
    del flush
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed steps for this long before the warm-up steps")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=25.0,
                    help="seconds of float64 oracle work for cpu_baseline (the whole step fits in about 20)")
    ap.add_argument("--skip-configs", action="store_true",
                    help="skip the per-configuration measurements of the other workloads")
    ap.add_argument("--only", choices=["select", "gather", "attn", "attn_dense", "attn_sparse", "scatter"],
                    help="time only this operation of the step (for counter runs); prints one line")
    ap.add_argument("--select-only", choices=["sparse_32k", "sparse_128k"],
                    help="time bd_select alone on one sparse workload (for profiling)")
    ap.add_argument("--pool-only", choices=["sparse_32k", "sparse_128k"],
                    help="time the T denoising attentions over one sparse workload's pool alone "
                         "(select and gather run once before, untimed; for profiling)")
    ap.add_argument("--producer-only", action="store_true",
                    help="time only the fused producer and its unfused sequence; prints one JSON line")
    ap.add_argument("--copy-probe", type=int, metavar="MB",
                    help="run a plain device copy of MB megabytes 5 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from sparse_kv_cache_bd_amd import bdattn as bd
    from sparse_kv_cache_bd_amd.pipeline import BlockDiffusionStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    bd.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy probe: 5 copies of {n * 4} bytes", flush=True)
        return
    if args.producer_only:
        print(json.dumps({"producer_serving_mix": bench_producer(bd, dev, args.steps)}), flush=True)
        return
    if args.select_only:
        wl = getattr(synth, args.select_only)()
        Kc, Qsel = wl.Kc.to(dev), wl.Qsel.to(dev)
        s_len, k_sel = wl.s_len.to(dev), wl.k_sel.to(dev)
        idx = torch.empty((wl.B, wl.Hkv, wl.k_max), dtype=torch.int32, device=dev)
        ws = bd.workspace(bd.select_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.d, wl.s_max, wl.k_max), dev)
        f = lambda: bd.select(Qsel, Kc, s_len, wl.s_max, k_sel, wl.k_max, wl.sm_scale, idx_out=idx, ws=ws)
        for _ in range(args.warmup):
            f()
        ms = time_calls(f, args.steps, 0, settle_ms=args.settle_ms)
        print(f"select {args.select_only}: {ms * 1e3:.1f} us per call over {args.steps} calls", flush=True)
        return
    if args.pool_only:
        wl = getattr(synth, args.pool_only)()
        Kc, Vc, Qsel = wl.Kc.to(dev), wl.Vc.to(dev), wl.Qsel.to(dev)
        s_len, k_sel = wl.s_len.to(dev), wl.k_sel.to(dev)
        B, Hkv, d, k_max, s_max = wl.B, wl.Hkv, wl.d, wl.k_max, wl.s_max
        idx = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=dev)
        ws = bd.workspace(bd.select_workspace_size(B, wl.Hq, Hkv, d, s_max, k_max), dev)
        pool_k = torch.zeros((B, k_max, Hkv, d), dtype=Kc.dtype, device=dev)
        pool_v = torch.zeros_like(pool_k)
        bd.select(Qsel, Kc, s_len, s_max, k_sel, k_max, wl.sm_scale, idx_out=idx, ws=ws)
        bd.gather(Kc, Vc, idx, k_sel, pool_k, pool_v)
        steps_q = [x.to(dev) for x in wl.extra["step_q"]]
        steps_kv = [(a.to(dev), b.to(dev)) for a, b in wl.extra["step_kv"]]
        outb = torch.empty_like(steps_q[0])
        ws_a = bd.workspace(bd.attn_workspace_size(Qsel.dtype, B, wl.Hq, Hkv, d, wl.q, B, k_max), dev)

        def f():
            for st in range(wl.T):
                wk, wv = steps_kv[st]
                bd.attn_packed(steps_q[st], pool_k, pool_v, k_sel, k_max, wk, wv, wl.bl,
                               wl.sm_scale, out=outb, ws=ws_a)
        for _ in range(args.warmup):
            f()
        ms = time_calls(f, args.steps, 0, settle_ms=args.settle_ms)
        print(f"pool attention {args.pool_only}: {ms * 1e3 / wl.T:.2f} us per denoising step "
              f"over {args.steps} x {wl.T} steps", flush=True)
        return
    log("generating the serving-mix workload")
    wl = synth.serving_mix(seed=args.seed)
    Kc, Vc, Q, o = (x.to(dev) for x in (wl.Kc, wl.Vc, wl.Q, wl.o))
    dense_pmax = int(wl.o[wl.dense_rows.long()].max()) if len(wl.dense_rows) else 0
    step = BlockDiffusionStep(Kc, Vc, Q, o, wl.bl, wl.sm_scale, sparse_rows=wl.sparse_rows,
                              dense_rows=wl.dense_rows, s_len=wl.s_len, k_sel=wl.k_sel,
                              p_max_dense=dense_pmax, k_max=wl.k_max, s_max=wl.s_max)
    work = step_work(wl)
    log(f"rows={wl.B} dense={step.n_dense} sparse={step.n_sparse} warmup={args.warmup} steps={args.steps}")
    # settle phase: the step repeated for a fixed wall time (batches of 10
    # steps, then a synchronisation), so the timed steps start at steady state
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            step.run()
        settle_steps += 10
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    if args.only:
        ms = time_calls(getattr(step, args.only), args.steps, 0, settle_ms=0)
        print(f"{args.only}: {ms * 1e3:.1f} us per call over {args.steps} calls", flush=True)
        return

    # timed region: exactly K steps and nothing else on the stream (an event
    # recorded between two kernels adds a gap of its own, so the per-operation
    # events are taken in a separate pass below)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step.run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ev_step = ev0.elapsed_time(ev1) / args.steps

    # per-operation pass: the same K steps with an event after every operation
    ops = BlockDiffusionStep.OPS
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        e = ev[s]
        e[0].record()
        for i, name in enumerate(ops):
            getattr(step, name)()
            e[i + 1].record()
    torch.cuda.synchronize()
    op_ms = {name: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
             for i, name in enumerate(ops)}
    ev_step_ops = sum(ev[s][0].elapsed_time(ev[s][-1]) for s in range(args.steps)) / args.steps
    log(f"step {ms_step:.3f} ms (events {ev_step:.3f} ms); with an event after every operation "
        f"{ev_step_ops:.3f} ms: " + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in op_ms.items()))

    attn_flop = work["attn_dense_flop"] + work["attn_sparse_flop"]
    attn_bytes = work["attn_dense_bytes"] + work["attn_sparse_bytes"]
    value = attn_flop / (ms_step * 1e-3) / 1e12
    # the two row kinds as separate launches (reference figures)
    ms_dense = time_calls(step.attn_dense, args.steps)
    ms_sparse = time_calls(step.attn_sparse, args.steps)

    def rate(num, ms, scale):
        return num / (ms * 1e-3) / scale if ms > 0 else None

    bd_ = {}
    tf_a = rate(attn_flop, op_ms["attn"], 1e12)
    tf_d = rate(work["attn_dense_flop"], ms_dense, 1e12)
    tf_s = rate(work["attn_sparse_flop"], ms_sparse, 1e12)
    gb_sel = rate(work["select_bytes"], op_ms["select"], 1e9)
    gb_gat = rate(work["gather_bytes"], op_ms["gather"], 1e9)
    gb_sca = rate(work["scatter_bytes"], op_ms["scatter"], 1e9)
    bd_["attn"] = {"us": round(op_ms["attn"] * 1e3, 2), "TFLOP/s": round(tf_a, 2),
                   "frac_mfma_peak": round(tf_a / PEAK_BF16_TFLOPS, 4),
                   "gflop": round(attn_flop / 1e9, 3)}
    bd_["attn_dense"] = {"us": round(ms_dense * 1e3, 2), "TFLOP/s": round(tf_d, 2),
                         "frac_mfma_peak": round(tf_d / PEAK_BF16_TFLOPS, 4),
                         "gflop": round(work["attn_dense_flop"] / 1e9, 3), "launch": "separate"}
    bd_["attn_sparse"] = {"us": round(ms_sparse * 1e3, 2), "TFLOP/s": round(tf_s, 2),
                          "frac_mfma_peak": round(tf_s / PEAK_BF16_TFLOPS, 4),
                          "gflop": round(work["attn_sparse_flop"] / 1e9, 3), "launch": "separate"}
    bd_["select"] = {"us": round(op_ms["select"] * 1e3, 2), "GB/s": round(gb_sel, 1),
                     "frac_hbm_peak": round(gb_sel / PEAK_HBM_GBS, 4),
                     "mb": round(work["select_bytes"] / 1e6, 2)}
    bd_["gather"] = {"us": round(op_ms["gather"] * 1e3, 2), "GB/s": round(gb_gat, 1),
                     "frac_hbm_peak": round(gb_gat / PEAK_HBM_GBS, 4),
                     "mb": round(work["gather_bytes"] / 1e6, 2)}
    bd_["scatter"] = {"us": round(op_ms["scatter"] * 1e3, 2), "GB/s": round(gb_sca, 1),
                      "frac_hbm_peak": round(gb_sca / PEAK_HBM_GBS, 4),
                      "mb": round(work["scatter_bytes"] / 1e6, 2)}

    traffic = traffic_for_attention()
    roof = {"bound": "mfma", "kernel": "attn_mfma_kernel<8, 4, false, false> (dense and sparse rows, one launch)",
            "achieved": round(tf_a, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf_a / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
            "algorithmic_bytes": attn_bytes,
            "intensity_flop_per_byte": round(attn_flop / attn_bytes, 1)}

    n_dense, n_sparse = step.n_dense, step.n_sparse
    block_table = None
    if not args.skip_configs:
        log("block table over the dense rows")
        block_table = bench_block_table(bd, wl, Kc, Vc, Q, dense_pmax, ms_dense, args.steps)
    configs = None
    if not args.skip_configs:
        del step, Kc, Vc, Q, o
        torch.cuda.empty_cache()
        configs = bench_configs(dev)
        configs["block_table_serving_mix_dense"] = block_table
        log("HBM reference: torch copy / sum / fill of 1 GiB")
        configs["hbm_reference"] = hbm_reference(dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on a bounded sample (cpu_baseline)")
        cpu = cpu_baseline(wl, args.cpu_budget)

    res = {"metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_ms": round(settle_ms, 1),
           "settle_steps": settle_steps, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "serving_mix", "rows": wl.B, "dense_rows": n_dense,
                      "sparse_rows": n_sparse, "prefix": "log-uniform 1K-16K",
                      "bl": wl.bl, "W": wl.W, "q": wl.q, "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d,
                      "C": wl.C, "budget": 0.05, "seed": args.seed},
           "roofline": roof, "cpu_baseline": cpu, "breakdown": bd_, "configs": configs}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
