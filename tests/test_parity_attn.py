"""GPU parity of bd_attn_packed against the float64 oracle.

Cases span several key tiles with ragged ends, both the split-KV and the
single-chunk plans, every built GQA group size, window shapes where q or
bl are not multiples of the 32-query tile, NaN sentinels in rows that must
never be read, row subsets, sharp logits, and a closed-form check of the
block-causal window (slot-tagged values with uniform attention).
"""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import check_attention, note
from oracle import bd_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


def _cache_case(seed, B, C, Hq, Hkv, d, bl, W, o, dtype=torch.bfloat16, qk_scale=None,
                v_scale=None):
    rs = np.random.default_rng(seed)
    q = W * bl
    t = C - q
    s = 1.0 / math.sqrt(d) if qk_scale is None else qk_scale
    vs = 1.0 / math.sqrt(d) if v_scale is None else v_scale
    K = rs.standard_normal((B, C, Hkv, d)).astype(np.float32) * s
    V = rs.standard_normal((B, C, Hkv, d)).astype(np.float32) * vs
    for b in range(B):
        K[b, o[b]:t] = np.nan
        V[b, o[b]:t] = np.nan
    Q = rs.standard_normal((B, q, Hq, d)).astype(np.float32) * s
    return (torch.from_numpy(Q).to(dtype), torch.from_numpy(K).to(dtype),
            torch.from_numpy(V).to(dtype), q, t)


def _run_cache(bd, Q, K, V, o, bl, scale, row_ids=None, lse=False):
    q = Q.shape[1]
    t = K.shape[1] - q
    Qd, Kd, Vd = Q.cuda(), K.cuda(), V.cuda()
    out = torch.full_like(Qd, 5.0)
    L = torch.full((Q.shape[0], Q.shape[2], q), 5.0, device="cuda") if lse else None
    rid = None if row_ids is None else torch.tensor(row_ids, dtype=torch.int32).cuda()
    bd.attn_packed(Qd, Kd, Vd, torch.tensor(o, dtype=torch.int32).cuda(), int(max(o)),
                   Kd[:, t:], Vd[:, t:], bl, scale, out=out, lse=L, row_ids=rid)
    torch.cuda.synchronize()
    return out, L


@pytest.mark.parametrize("G,Hkv,W,bl,o,d", [
    (4, 2, 2, 32, [0, 37, 300], 128),       # zero, ragged, several tiles
    (1, 4, 2, 32, [64, 129], 128),
    (2, 3, 3, 16, [100, 7], 128),           # q = 48: partial query tile
    (8, 1, 1, 64, [500], 128),              # bl = 64: two query tiles, one slot
    (4, 2, 5, 8, [33, 200, 64], 128),       # bl = 8: slots inside a query tile
    (4, 2, 4, 32, [1000, 16], 128),
    (4, 2, 2, 32, [70, 300], 64),           # general path (bf16, d = 64)
])
def test_cache_attention(bd, G, Hkv, W, bl, o, d):
    note(f"attn cache G={G} Hkv={Hkv} W={W} bl={bl} o={o} d={d}")
    B = len(o)
    Hq = G * Hkv
    C = max(o) + W * bl + 40
    Q, K, V, q, t = _cache_case(G * 100 + W, B, C, Hq, Hkv, d, bl, W, o)
    scale = 1.0 / math.sqrt(d)
    out, L = _run_cache(bd, Q, K, V, o, bl, scale, lse=True)
    ref, ref_lse = orc.cache_attention_eq6(Q, K, V, o, bl, scale)
    check_attention(out, ref, torch.bfloat16, label="cache")
    np.testing.assert_allclose(L.cpu().numpy(), ref_lse, atol=2e-3, rtol=1e-3)


@pytest.mark.parametrize("B,o_max,W", [(1, 5000, 1), (2, 2300, 2), (16, 900, 4)])
def test_split_and_single_chunk_plans(bd, B, o_max, W):
    """1-2 rows force the split-KV plan with a combine; 16 rows x 8 KV heads
    x 4 query tiles keep one chunk per unit."""
    note(f"attn plans B={B} o_max={o_max} W={W}")
    Hkv, G, d, bl = 8, 4, 128, 32
    rs = np.random.default_rng(B)
    o = list(rs.integers(1, o_max, size=B))
    o[0] = o_max
    C = o_max + W * bl
    Q, K, V, q, t = _cache_case(B + 7, B, C, G * Hkv, Hkv, d, bl, W, o)
    need = bd.attn_workspace_size(torch.bfloat16, B, G * Hkv, Hkv, d, q, B, max(o))
    assert (need > 0) == (B < 16)
    out, L = _run_cache(bd, Q, K, V, o, bl, 1.0 / math.sqrt(d), lse=True)
    ref, ref_lse = orc.cache_attention_eq6(Q, K, V, o, bl, 1.0 / math.sqrt(d))
    check_attention(out, ref, torch.bfloat16, label="plan")
    np.testing.assert_allclose(L.cpu().numpy(), ref_lse, atol=2e-3, rtol=1e-3)


@pytest.mark.parametrize("n_rows", [200, 300])
def test_many_rows_longest_first(bd, n_rows):
    """More work items than the GPU holds: the planner kernel ranks the rows
    and blocks take them longest first (with split prefixes at 200 rows, one
    chunk per unit at 300).  The order is a schedule only, so every row must
    match."""
    G, Hkv, W, bl, d = 4, 2, 1, 32, 128
    rs = np.random.default_rng(n_rows)
    o = [int(v) for v in rs.integers(0, 400, size=n_rows)]
    o[int(rs.integers(0, n_rows))] = 0
    note(f"attn many rows n={n_rows} o in [{min(o)}, {max(o)}]")
    C = max(o) + W * bl + 8
    Q, K, V, q, t = _cache_case(700 + n_rows, n_rows, C, G * Hkv, Hkv, d, bl, W, o)
    ws = bd.attn_workspace_size(bd.BD_BF16, n_rows, G * Hkv, Hkv, d, q, n_rows, max(o))
    # the planner's order buffer (n_rows int32), plus split partials at 200 rows
    order = ((n_rows * 4 + 255) // 256) * 256
    assert (ws > order) if n_rows == 200 else (ws == order)
    scale = 1.0 / math.sqrt(d)
    out, _ = _run_cache(bd, Q, K, V, o, bl, scale)
    pick = sorted(set(rs.choice(n_rows, 20, replace=False).tolist() +
                      [int(np.argmax(o)), int(np.argmin(o))]))
    ref, _ = orc.cache_attention_eq6(Q[pick], K[pick], V[pick], [o[i] for i in pick], bl, scale)
    check_attention(out[pick], ref, torch.bfloat16, label=f"many rows {n_rows}")


def test_sharp_logits(bd):
    """Unscaled N(0,1) Q, K, V with sm_scale = 1: peaked softmax."""
    note("attn sharp logits")
    o = [300, 65]
    Q, K, V, q, t = _cache_case(3, 2, 500, 8, 2, 128, 32, 2, o, qk_scale=1.0, v_scale=1.0)
    Q = Q * 0.35
    out, _ = _run_cache(bd, Q, K, V, o, 32, 1.0)
    ref, _ = orc.cache_attention_eq6(Q, K, V, o, 32, 1.0)
    check_attention(out, ref, torch.bfloat16, label="sharp")


def test_slot_tagged_window_closed_form(bd):
    """Q = 0 (uniform attention), prefix V = 0 and window V of slot s equal to
    s+1: query i averages (w // bl + 1) over w < lim(i), so
    O = sum_{w<lim} (w//bl + 1) / (P + lim).  A leak across slots changes it."""
    note("attn slot-tagged window")
    B, Hkv, G, d, bl, W = 2, 2, 4, 128, 32, 4
    q = W * bl
    P = [96, 0]
    C = 96 + q + 32
    t = C - q
    K = torch.randn((B, C, Hkv, d)).bfloat16()
    V = torch.zeros((B, C, Hkv, d))
    for w in range(q):
        V[:, t + w] = w // bl + 1
    V = V.bfloat16()
    Q = torch.zeros((B, q, G * Hkv, d)).bfloat16()
    out, _ = _run_cache(bd, Q, K, V, P, bl, 0.1)
    g = out.cpu().float().numpy()
    for b in range(B):
        for i in range(q):
            lim = (i // bl + 1) * bl
            want = sum(w // bl + 1 for w in range(lim)) / (P[b] + lim)
            assert np.allclose(g[b, i], want, rtol=8e-3), (b, i, g[b, i, 0, 0], want)


def test_row_subset_untouched(bd):
    note("attn row_ids subset")
    o = [200, 90, 310, 40]
    Q, K, V, q, t = _cache_case(9, 4, 420, 32, 8, 128, 32, 2, o)
    out, _ = _run_cache(bd, Q, K, V, o, 32, 0.09, row_ids=[2, 0, 77])
    ref, _ = orc.cache_attention_eq6(Q, K, V, o, 32, 0.09)
    check_attention(out, ref, torch.bfloat16, rows=[0, 2], label="subset")
    g = out.cpu().float()
    assert (g[[1, 3]] == 5.0).all()


def test_pool_form_with_nan_past_budget(bd):
    """Sparse call: prefix = pool with k_b valid entries, NaN past them."""
    note("attn pool form")
    rs = np.random.default_rng(21)
    B, Hkv, G, d, bl, W, kmax = 3, 8, 4, 128, 32, 1, 400
    q = W * bl
    kb = np.array([400, 123, 0], np.int32)
    pool_k = rs.standard_normal((B, kmax + 8, Hkv, d)).astype(np.float32) / math.sqrt(d)
    pool_v = rs.standard_normal((B, kmax + 8, Hkv, d)).astype(np.float32)
    for b in range(B):
        pool_k[b, kb[b]:] = np.nan
        pool_v[b, kb[b]:] = np.nan
    wk = rs.standard_normal((B, q, Hkv, d)).astype(np.float32) / math.sqrt(d)
    wv = rs.standard_normal((B, q, Hkv, d)).astype(np.float32)
    Q = rs.standard_normal((B, q, G * Hkv, d)).astype(np.float32) / math.sqrt(d)
    T = [torch.from_numpy(x).bfloat16() for x in (Q, pool_k, pool_v, wk, wv)]
    Qd, pkd, pvd, wkd, wvd = (x.cuda() for x in T)
    out = bd.attn_packed(Qd, pkd, pvd, torch.from_numpy(kb).cuda(), kmax, wkd, wvd, bl,
                         1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    ref, _ = orc.block_attention(*T[:3], kb, T[3], T[4], bl, 1.0 / math.sqrt(d))
    check_attention(out, ref, torch.bfloat16, label="pool")


def test_pool_long_ragged_combine_rounds(bd):
    """Pool rows of 16000 and 5000 keys with 4 KV heads and q = 32: the plan
    cuts them into 256-key chunks (63 and 20), so the combine takes its
    32-partials-per-round form, in two rounds for the long row and one
    partly filled round for the short one."""
    note("attn pool long ragged combine rounds")
    rs = np.random.default_rng(33)
    B, Hkv, G, d, bl, W = 2, 4, 4, 128, 32, 1
    q = W * bl
    kb = [16000, 5000]
    kmax = max(kb)
    PK, PV = _pool_case(rs, B, kmax + 8, Hkv, d, kb, torch.bfloat16)
    wk = torch.from_numpy(rs.standard_normal((B, q, Hkv, d)).astype(np.float32) / math.sqrt(d)).bfloat16()
    wv = torch.from_numpy(rs.standard_normal((B, q, Hkv, d)).astype(np.float32) / math.sqrt(d)).bfloat16()
    Q = torch.from_numpy(rs.standard_normal((B, q, G * Hkv, d)).astype(np.float32) / math.sqrt(d)).bfloat16()
    need = bd.attn_workspace_size(torch.bfloat16, B, G * Hkv, Hkv, d, q, B, kmax)
    # 63 chunks of bf16 partial O rows (2 bytes per element) for the long row
    assert need >= B * Hkv * 63 * 128 * d * 2, "plan does not split into 256-key chunks"
    L = torch.full((B, G * Hkv, q), 5.0, device="cuda")
    out = bd.attn_packed(Q.cuda(), PK.cuda(), PV.cuda(), torch.tensor(kb, dtype=torch.int32).cuda(), kmax,
                         wk.cuda(), wv.cuda(), bl, 1.0 / math.sqrt(d), lse=L)
    torch.cuda.synchronize()
    ref, ref_lse = orc.block_attention(Q, PK, PV, kb, wk, wv, bl, 1.0 / math.sqrt(d))
    check_attention(out, ref, torch.bfloat16, label="pool rounds")
    np.testing.assert_allclose(L.cpu().numpy(), ref_lse, atol=2e-3, rtol=1e-3)


@pytest.mark.parametrize("d,G", [(64, 1), (128, 4), (64, 2)])
def test_fp32_general_path(bd, d, G):
    note(f"attn fp32 d={d} G={G}")
    o = [256, 31]
    Q, K, V, q, t = _cache_case(d + G, 2, 330, 2 * G, 2, d, 32, 1, o, dtype=torch.float32)
    out, L = _run_cache(bd, Q, K, V, o, 32, 1.0 / math.sqrt(d), lse=True)
    ref, ref_lse = orc.cache_attention_eq6(Q, K, V, o, 32, 1.0 / math.sqrt(d))
    check_attention(out, ref, torch.float32, label="fp32")
    np.testing.assert_allclose(L.cpu().numpy(), ref_lse, atol=1e-5, rtol=1e-5)


def test_fp32_general_path_many_blocks(bd):
    """256 blocks (8 rows x 32 query heads): the general path with one key
    group per block; the small launches above take 2 or 4 key groups."""
    note("attn fp32 general path, 256 blocks")
    o = [300, 0, 45, 129, 77, 256, 5, 190]
    Q, K, V, q, t = _cache_case(41, 8, 340, 32, 8, 64, 32, 1, o, dtype=torch.float32)
    out, L = _run_cache(bd, Q, K, V, o, 32, 0.125, lse=True)
    ref, ref_lse = orc.cache_attention_eq6(Q, K, V, o, 32, 0.125)
    check_attention(out, ref, torch.float32, label="fp32 many blocks")
    np.testing.assert_allclose(L.cpu().numpy(), ref_lse, atol=1e-5, rtol=1e-5)


def test_fp32_general_path_split_prefix(bd):
    """Few general-path blocks over long ragged prefixes: the prefix is cut
    into 32-key chunks (dozens per row), each writing an fp32 partial, and
    the combine merges them; an empty prefix and a one-chunk row are written
    directly."""
    note("attn fp32 general path, split prefix")
    o = [2000, 0, 777, 19]
    Q, K, V, q, t = _cache_case(77, 4, 2100, 2, 2, 128, 32, 2, o, dtype=torch.float32)
    out, L = _run_cache(bd, Q, K, V, o, 32, 1.0 / math.sqrt(128), lse=True)
    ref, ref_lse = orc.cache_attention_eq6(Q, K, V, o, 32, 1.0 / math.sqrt(128))
    check_attention(out, ref, torch.float32, label="fp32 split prefix")
    np.testing.assert_allclose(L.cpu().numpy(), ref_lse, atol=1e-5, rtol=1e-5)
    plan_bytes = bd.attn_workspace_size(torch.float32, 4, 2, 2, 128, q, 4, max(o))
    assert plan_bytes > 0          # the plan splits this launch


def test_tiny_dense_config(bd):
    """The tiny fp32 configuration: 1 row, 4/4 heads, d = 64, prefix 256,
    W = 1, plus the scatter of the 32 new KV rows."""
    note("config tiny_dense")
    wl = synth.tiny_dense()
    out, L = _run_cache(bd, wl.Q, wl.Kc, wl.Vc, wl.o.tolist(), wl.bl, wl.sm_scale, lse=True)
    ref, ref_lse = orc.cache_attention_eq6(wl.Q, wl.Kc, wl.Vc, wl.o, wl.bl, wl.sm_scale)
    check_attention(out, ref, torch.float32, label="tiny_dense")
    np.testing.assert_allclose(L.cpu().numpy(), ref_lse, atol=1e-5, rtol=1e-5)


def _pool_case(rs, B, P, Hkv, d, k, dtype):
    """Pool [B, P, Hkv, d] whose entries at or past each row's k_b hold NaN."""
    s = 1.0 / math.sqrt(d)
    PK = rs.standard_normal((B, P, Hkv, d)).astype(np.float32) * s
    PV = rs.standard_normal((B, P, Hkv, d)).astype(np.float32) * s
    for b in range(B):
        PK[b, k[b]:] = np.nan
        PV[b, k[b]:] = np.nan
    return torch.from_numpy(PK).to(dtype), torch.from_numpy(PV).to(dtype)


@pytest.mark.parametrize("B,o_max,k_max,W,d,G,dtype", [
    (6, 3000, 400, 4, 128, 4, torch.bfloat16),    # longest-first order, one chunk per unit
    (3, 1500, 300, 1, 128, 4, torch.bfloat16),    # few units: split prefixes + combine
    (4, 700, 200, 2, 64, 2, torch.float32),       # general path
])
def test_dual_sources_match_each_source(bd, B, o_max, k_max, W, d, G, dtype):
    """bd_attn_packed_dual: rows of list a over the cache (FlowBlock Eq. (6)),
    rows of list b over a pool (HERALD's denoising attention), one row in
    neither list (left untouched); each row matches the oracle for its own
    source, and the LSE too."""
    note(f"dual B={B} o_max={o_max} k_max={k_max} W={W} d={d} G={G} {dtype}")
    rs = np.random.default_rng(70 + B)
    Hkv, bl = 2, 32
    q = W * bl
    C = o_max + 64 + q
    o = [int(x) for x in rs.integers(1, o_max, size=B)]
    o[0] = o_max
    kb = [int(x) for x in rs.integers(1, k_max, size=B)]
    kb[-1] = k_max
    Q, K, V, q, t = _cache_case(80 + B, B, C, G * Hkv, Hkv, d, bl, W, o, dtype=dtype)
    PK, PV = _pool_case(rs, B, k_max + 32, Hkv, d, kb, dtype)
    rows_a = [b for b in range(B - 1) if b % 2 == 0]
    rows_b = [b for b in range(B - 1) if b % 2 == 1]
    Qd, Kd, Vd, PKd, PVd = Q.cuda(), K.cuda(), V.cuda(), PK.cuda(), PV.cuda()
    out = torch.full_like(Qd, 5.0)
    L = torch.full((B, G * Hkv, q), 5.0, device="cuda")
    i32 = lambda x: torch.tensor(x, dtype=torch.int32).cuda()
    bd.attn_packed_dual(Qd, (i32(rows_a), Kd, Vd, i32(o), max(o)),
                        (i32(rows_b), PKd, PVd, i32(kb), k_max),
                        Kd[:, t:], Vd[:, t:], bl, 1.0 / math.sqrt(d), out=out, lse=L)
    torch.cuda.synchronize()
    ref_a, lse_a = orc.block_attention(Q, K, V, o, K[:, t:], V[:, t:], bl, 1.0 / math.sqrt(d),
                                       rows=rows_a)
    ref_b, lse_b = orc.block_attention(Q, PK, PV, kb, K[:, t:], V[:, t:], bl, 1.0 / math.sqrt(d),
                                       rows=rows_b)
    check_attention(out, ref_a, dtype, rows=rows_a, label="dual list a")
    check_attention(out, ref_b, dtype, rows=rows_b, label="dual list b")
    Lh = L.cpu().numpy()
    tol = (2e-3, 1e-3) if dtype == torch.bfloat16 else (1e-5, 1e-5)
    np.testing.assert_allclose(Lh[rows_a], lse_a[rows_a], atol=tol[0], rtol=tol[1])
    np.testing.assert_allclose(Lh[rows_b], lse_b[rows_b], atol=tol[0], rtol=tol[1])
    assert torch.all(out[B - 1] == 5.0) and torch.all(L[B - 1] == 5.0), "unlisted row written"


def test_dual_equals_two_single_calls(bd):
    """The one-launch call gives bit-identical outputs to two bd_attn_packed
    calls (each row's arithmetic does not depend on the other list).  Prefixes
    stay at or below 256 keys, so no call splits them into chunks and every
    call runs the same per-row plan."""
    note("dual vs two single calls")
    rs = np.random.default_rng(91)
    B, Hkv, G, d, bl, W = 8, 2, 4, 128, 32, 4
    q = W * bl
    o = [int(x) for x in rs.integers(100, 257, size=B)]
    kb = [int(x) for x in rs.integers(50, 257, size=B)]
    Q, K, V, q, t = _cache_case(92, B, max(o) + 64 + q, G * Hkv, Hkv, d, bl, W, o)
    PK, PV = _pool_case(rs, B, 288, Hkv, d, kb, torch.bfloat16)
    Qd, Kd, Vd, PKd, PVd = Q.cuda(), K.cuda(), V.cuda(), PK.cuda(), PV.cuda()
    i32 = lambda x: torch.tensor(x, dtype=torch.int32).cuda()
    ra, rb = [0, 2, 3, 5, 6], [1, 4, 7]
    one = bd.attn_packed_dual(Qd, (i32(ra), Kd, Vd, i32(o), max(o)), (i32(rb), PKd, PVd, i32(kb), 256),
                              Kd[:, t:], Vd[:, t:], bl, 0.1)
    two = torch.empty_like(Qd)
    bd.attn_packed(Qd, Kd, Vd, i32(o), max(o), Kd[:, t:], Vd[:, t:], bl, 0.1, out=two, row_ids=i32(ra))
    bd.attn_packed(Qd, PKd, PVd, i32(kb), 256, Kd[:, t:], Vd[:, t:], bl, 0.1, out=two, row_ids=i32(rb))
    torch.cuda.synchronize()
    assert torch.equal(one, two)
