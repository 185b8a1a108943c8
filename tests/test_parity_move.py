"""GPU parity of the KV movement kernels and the mask predicate: bit-exact
against the oracle (FlowBlock review Eq. (6), Eq. (7); HERALD Sec. IV-B3)."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import bits, note
from oracle import bd_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("dtype,L,B,C,Hkv,d,q,alias", [
    ("bf16", 1, 4, 256, 8, 128, 64, True),
    ("bf16", 3, 5, 300, 2, 64, 40, True),
    ("f32", 1, 1, 512, 4, 64, 32, True),
    ("f32", 2, 3, 200, 3, 128, 17, False),
    ("bf16", 1, 2, 128, 1, 8, 33, False),
])
def test_scatter_bitexact(bd, dtype, L, B, C, Hkv, d, q, alias):
    note(f"scatter {dtype} L={L} B={B} C={C} Hkv={Hkv} d={d} q={q} alias={alias}")
    rs = np.random.default_rng(C + q)
    t = C - q
    data = torch.from_numpy(rs.standard_normal((L, B, C, Hkv, d)).astype(np.float32)).to(DT[dtype])
    present = data if alias else torch.from_numpy(
        rs.standard_normal((L, B, C, Hkv, d)).astype(np.float32)).to(DT[dtype])
    o = rs.integers(0, t - q + 1, size=B)
    if alias:
        o[0] = t                          # writes the tail onto itself
    if B > 2:
        o[1] = C                          # out of range: the row is skipped
    o_t = torch.from_numpy(o.astype(np.int32))
    dk, dv = data.cuda(), (data * 2).cuda()
    pk, pv = (dk, dv) if alias else (present.cuda(), (present * 2).cuda())
    bd.kv_scatter(pk, pv, dk, dv, o_t.cuda(), t, q)
    torch.cuda.synchronize()
    valid = np.array([ob + q <= C for ob in o])
    rows = np.nonzero(valid)[0]
    ref_k = orc.kv_scatter(bits(present), bits(data), o, t, q, rows=rows)
    ref_v = orc.kv_scatter(bits(present * 2), bits(data * 2), o, t, q, rows=rows)
    assert np.array_equal(bits(dk), ref_k)
    assert np.array_equal(bits(dv), ref_v)


def test_scatter_row_subset(bd):
    note("scatter row_ids subset")
    rs = np.random.default_rng(5)
    L, B, C, Hkv, d, q = 1, 6, 160, 4, 128, 32
    t = C - q
    data = torch.from_numpy(rs.standard_normal((L, B, C, Hkv, d)).astype(np.float32)).bfloat16()
    o = rs.integers(0, t - q + 1, size=B).astype(np.int32)
    rows = np.array([4, 1, 9, -1], dtype=np.int32)      # 9 and -1 are skipped
    dk = data.cuda()
    bd.kv_scatter(dk, None, dk, None, torch.from_numpy(o).cuda(), t, q,
                  row_ids=torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    ref = orc.kv_scatter(bits(data), bits(data), o, t, q, rows=[4, 1])
    assert np.array_equal(bits(dk), ref)


@pytest.mark.parametrize("dtype,B,S,Hkv,d,kmax", [
    ("bf16", 3, 1000, 8, 128, 70),
    ("f32", 2, 300, 4, 64, 129),
    ("bf16", 1, 50, 2, 64, 50),
])
def test_gather_bitexact(bd, dtype, B, S, Hkv, d, kmax):
    note(f"gather {dtype} B={B} S={S} Hkv={Hkv} d={d} kmax={kmax}")
    rs = np.random.default_rng(S)
    src_k = torch.from_numpy(rs.standard_normal((B, S, Hkv, d)).astype(np.float32)).to(DT[dtype])
    src_v = -src_k
    k_cnt = rs.integers(0, kmax + 1, size=B).astype(np.int32)
    k_cnt[0] = kmax
    idx = np.full((B, Hkv, kmax), -1, np.int32)
    for b in range(B):
        for h in range(Hkv):
            idx[b, h, :k_cnt[b]] = np.sort(rs.choice(S, k_cnt[b], replace=False))
    pool_k = torch.full((B, kmax + 3, Hkv, d), 7.0, dtype=DT[dtype])
    pool_v = torch.full((B, kmax + 3, Hkv, d), -7.0, dtype=DT[dtype])
    gk, gv = pool_k.cuda(), pool_v.cuda()
    bd.gather(src_k.cuda(), src_v.cuda(), torch.from_numpy(idx).cuda(),
              torch.from_numpy(k_cnt).cuda(), gk, gv)
    torch.cuda.synchronize()
    assert np.array_equal(bits(gk), orc.gather(bits(src_k), idx, k_cnt, bits(pool_k)))
    assert np.array_equal(bits(gv), orc.gather(bits(src_v), idx, k_cnt, bits(pool_v)))


def test_scatter_gather_round_trip(bd):
    note("scatter then gather round trip")
    rs = np.random.default_rng(11)
    B, C, Hkv, d, q = 4, 512, 8, 128, 64
    t = C - q
    cache = torch.from_numpy(rs.standard_normal((B, C, Hkv, d)).astype(np.float32)).bfloat16().cuda()
    tail = cache[:, t:].clone()
    o = torch.tensor([0, 100, 300, 448], dtype=torch.int32)
    bd.kv_scatter(cache, None, cache, None, o.cuda(), t, q)
    idx = (o[:, None, None] + torch.arange(q)[None, None, :]).expand(B, Hkv, q).contiguous().int()
    pool = torch.zeros((B, q, Hkv, d), dtype=torch.bfloat16, device="cuda")
    bd.gather(cache, None, idx.cuda(), torch.full((B,), q, dtype=torch.int32).cuda(), pool, None)
    torch.cuda.synchronize()
    assert np.array_equal(bits(pool), bits(tail))


def test_mask_hook_hwp_diagram(bd, golden_dir):
    note("mask hook: FlowBlock packing diagram rows")
    with open(os.path.join(golden_dir, "hwp_diagram.json")) as f:
        gd = json.load(f)
    o = np.array([s["o"] for s in gd["sequences"]], np.int32)
    C, q, bl = 256, gd["q"], gd["bl"]
    m = bd.mask_materialize(len(o), C, q, bl, torch.from_numpy(o).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(m.cpu().numpy().astype(bool), orc.eq6_mask(C, q, bl, o))


@pytest.mark.parametrize("C,bl,W", [(128, 32, 1), (200, 8, 4), (97, 5, 3), (4096, 32, 2),
                                    (16640, 32, 4)])
def test_mask_hook_bitexact(bd, C, bl, W):
    note(f"mask hook C={C} bl={bl} W={W}")
    q = W * bl
    t = C - q
    rs = np.random.default_rng(C)
    o = np.concatenate([[0, t, 1], rs.integers(0, t + 1, size=5)]).astype(np.int32)
    m = bd.mask_materialize(len(o), C, q, bl, torch.from_numpy(o).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(m.cpu().numpy().astype(bool), orc.eq6_mask(C, q, bl, o))


def test_scatter_many_items_per_block(bd):
    """More work items than resident blocks (4 layers x 64 rows x 2 tensors
    x 16 chunks of 8 positions = 8192 > 2048): every block walks several
    items with the next item's loads in flight during the current stores."""
    note("scatter: 8192 items over 2048 blocks")
    rs = np.random.default_rng(77)
    L, B, C, Hkv, d, q = 4, 64, 300, 8, 128, 128
    t = C - q
    data = torch.from_numpy(rs.standard_normal((L, B, C, Hkv, d)).astype(np.float32)).bfloat16()
    o = rs.integers(0, t - q + 1, size=B).astype(np.int32)
    o[5] = -1                                        # skipped rows among the items
    o[6] = t                                         # identity write
    dk, dv = data.cuda(), (-data).cuda()
    bd.kv_scatter(dk, dv, dk, dv, torch.from_numpy(o).cuda(), t, q)
    torch.cuda.synchronize()
    rows = [b for b in range(B) if o[b] >= 0]
    assert np.array_equal(bits(dk), orc.kv_scatter(bits(data), bits(data), o, t, q, rows=rows))
    assert np.array_equal(bits(dv), orc.kv_scatter(bits(-data), bits(-data), o, t, q, rows=rows))


def _gather_case(B, S, Hkv, d, kmax, seed, empty_frac=0.0):
    rs = np.random.default_rng(seed)
    src_k = torch.from_numpy(rs.standard_normal((B, S, Hkv, d)).astype(np.float32)).bfloat16()
    k_cnt = rs.integers(1, kmax + 1, size=B).astype(np.int32)
    k_cnt[rs.random(B) < empty_frac] = 0
    idx = np.full((B, Hkv, kmax), -1, np.int32)
    for b in range(B):
        for h in range(Hkv):
            idx[b, h, :k_cnt[b]] = np.sort(rs.choice(S, k_cnt[b], replace=False))
    return src_k, k_cnt, idx


@pytest.mark.parametrize("B,S,Hkv,kmax,empty", [
    (8, 20000, 8, 3000, 0.0),       # 6016 items over 2048 blocks
    (300, 400, 2, 90, 0.9),         # mostly empty rows
    (4100, 40, 1, 8, 0.5),          # more rows than the LDS numbering: one block per row chunk
])
def test_gather_items_and_rows(bd, B, S, Hkv, kmax, empty):
    note(f"gather B={B} S={S} Hkv={Hkv} kmax={kmax} empty={empty}")
    src_k, k_cnt, idx = _gather_case(B, S, Hkv, 128, kmax, B + S, empty)
    pool = torch.full((B, kmax, Hkv, 128), 3.0, dtype=torch.bfloat16)
    gk, gv = pool.cuda(), (-pool).cuda()
    bd.gather(src_k.cuda(), (2 * src_k).cuda(), torch.from_numpy(idx).cuda(),
              torch.from_numpy(k_cnt).cuda(), gk, gv)
    torch.cuda.synchronize()
    assert np.array_equal(bits(gk), orc.gather(bits(src_k), idx, k_cnt, bits(pool)))
    assert np.array_equal(bits(gv), orc.gather(bits(2 * src_k), idx, k_cnt, bits(-pool)))


def test_gather_out_of_contract_values(bd):
    """Counts above k_max are clamped to k_max, negative counts gather
    nothing, and a slot whose index lies outside [0, S) keeps its value."""
    note("gather: clamped counts and out-of-range indices")
    B, S, Hkv, kmax = 4, 500, 2, 40
    src_k, _, _ = _gather_case(B, S, Hkv, 128, kmax, 9)
    rs = np.random.default_rng(10)
    idx = np.stack([np.stack([np.sort(rs.choice(S, kmax, replace=False)) for _ in range(Hkv)])
                    for _ in range(B)]).astype(np.int32)
    idx[0, 1, 3] = -1
    idx[1, 0, 7] = S
    idx[3, 1, 0] = 1 << 30
    k_cnt = np.array([kmax, kmax + 50, -4, 25], np.int32)
    pool = torch.full((B, kmax, Hkv, 128), 5.0, dtype=torch.bfloat16)
    gk = pool.cuda()
    bd.gather(src_k.cuda(), None, torch.from_numpy(idx).cuda(), torch.from_numpy(k_cnt).cuda(), gk, None)
    torch.cuda.synchronize()
    eff = np.clip(k_cnt, 0, kmax)
    safe = np.where((idx >= 0) & (idx < S), idx, 0)
    ref = orc.gather(bits(src_k), safe, eff, bits(pool))
    p0 = bits(pool)
    for b, h, j in ((0, 1, 3), (1, 0, 7), (3, 1, 0)):
        ref[b, j, h] = p0[b, j, h]                 # left unchanged
    assert np.array_equal(bits(gk), ref)
