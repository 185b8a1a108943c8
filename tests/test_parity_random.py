"""Seeded random shapes against the float64 oracle: attention (every window
mask, MFMA and general paths, cache form with NaN sentinels), selection and
multi-query selection (indices bit-exact on the GPU's scores, scores within
the stated bound), and the scatter/gather round trip.  Each case prints its
parameters before it runs."""
import math

import numpy as np
import pytest
import torch

from gpu_util import bits, check_attention, check_scores, note
from oracle import bd_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


def _attn_case(seed):
    rs = np.random.default_rng(1000 + seed)
    mfma = seed % 3 != 2
    d = 128 if mfma else int(rs.choice([64, 128]))
    dtype = torch.bfloat16 if mfma else (torch.float32 if seed % 2 else torch.bfloat16)
    G = int(rs.choice([1, 2, 4, 8])) if mfma else int(rs.choice([1, 2, 3]))
    Hkv = int(rs.integers(1, 4))
    bl = int(rs.choice([8, 16, 32, 64]))
    W = int(rs.integers(1, 5))
    B = int(rs.integers(1, 5))
    mode = ["block_causal", "isolated", "shared_first"][seed % 3]
    o = [int(v) for v in rs.integers(0, 700, size=B)]
    return rs, dict(d=d, dtype=dtype, G=G, Hkv=Hkv, bl=bl, W=W, B=B, mode=mode, o=o)


@pytest.mark.parametrize("seed", range(12))
def test_random_attention(bd, seed):
    rs, c = _attn_case(seed)
    note(f"random attention seed={seed} {c}")
    B, d, G, Hkv, bl, W, o = c["B"], c["d"], c["G"], c["Hkv"], c["bl"], c["W"], c["o"]
    q = W * bl
    C = max(o) + q + int(rs.integers(0, 50))
    t = C - q
    sc = 1.0 / math.sqrt(d)
    K = rs.standard_normal((B, C, Hkv, d)).astype(np.float32) * sc
    V = rs.standard_normal((B, C, Hkv, d)).astype(np.float32)
    for b in range(B):
        K[b, o[b]:t] = np.nan
        V[b, o[b]:t] = np.nan
    Q = rs.standard_normal((B, q, G * Hkv, d)).astype(np.float32) * sc * (3.0 if seed % 4 == 0 else 1.0)
    Qt, Kt, Vt = (torch.from_numpy(x).to(c["dtype"]) for x in (Q, K, V))
    Qd, Kd, Vd = Qt.cuda(), Kt.cuda(), Vt.cuda()
    L = torch.full((B, G * Hkv, q), 5.0, device="cuda")
    out = bd.attn_packed(Qd, Kd, Vd, torch.tensor(o, dtype=torch.int32).cuda(), max(max(o), 1),
                         Kd[:, t:], Vd[:, t:], bl, sc, lse=L, mask_mode=c["mode"])
    torch.cuda.synchronize()
    ref, ref_lse = orc.cache_attention_eq6(Qt, Kt, Vt, o, bl, sc, c["mode"])
    check_attention(out, ref, c["dtype"], label=f"seed {seed}")
    tol = (2e-3, 1e-3) if c["dtype"] == torch.bfloat16 else (1e-5, 1e-5)
    np.testing.assert_allclose(L.cpu().numpy(), ref_lse, atol=tol[0], rtol=tol[1])


@pytest.mark.parametrize("seed", range(8))
def test_random_selection(bd, seed):
    rs = np.random.default_rng(2000 + seed)
    B = int(rs.integers(1, 4))
    Hkv = int(rs.choice([1, 2, 4, 8]))
    G = int(rs.choice([1, 2, 4]))
    nq = int(rs.integers(1, 33))
    multi = seed % 2 == 1
    if multi:
        nq = min(nq, 128 // G)
    S = [int(v) for v in rs.integers(1, 9000, size=B)]
    k = [int(rs.integers(0, s + 40)) for s in S]
    note(f"random selection seed={seed} B={B} Hkv={Hkv} G={G} nq={nq} S={S} k={k} multi={multi}")
    d = 128
    C = max(S) + 8
    Q = rs.standard_normal((B, nq, G * Hkv, d)).astype(np.float32) / math.sqrt(d)
    K = rs.standard_normal((B, C, Hkv, d)).astype(np.float32) / math.sqrt(d)
    Qt, Kt = torch.from_numpy(Q).bfloat16(), torch.from_numpy(K).bfloat16()
    s_max, k_max = max(S), max(max(k), 1)
    sc_out = torch.full((B, Hkv, s_max), -3.0, device="cuda")
    fn = bd.select_multi if multi else bd.select
    idx = fn(Qt.cuda(), Kt.cuda(), torch.tensor(S, dtype=torch.int32).cuda(), s_max,
             torch.tensor(k, dtype=torch.int32).cuda(), k_max, 1.0 / math.sqrt(d), score_out=sc_out)
    torch.cuda.synchronize()
    sc = sc_out.cpu().double().numpy()
    if multi:
        ref = orc.multi_query_scores(Qt, Kt, S, 1.0 / math.sqrt(d))
    else:
        ref, _, _ = orc.selection_scores(orc.rep_query(Qt, "mean"), Kt, S, 1.0 / math.sqrt(d))
    check_scores(sc, ref, [s if kk > 0 else 0 for s, kk in zip(S, k)], f"seed {seed}")
    assert np.array_equal(idx.cpu().numpy(), orc.topk_select(sc, S, k, k_max))


@pytest.mark.parametrize("seed", range(4))
def test_random_scatter_gather_round_trip(bd, seed):
    """Scatter the window to random offsets, then gather positions o_b + delta
    back: the pool equals the window bit for bit; nothing else moved."""
    rs = np.random.default_rng(3000 + seed)
    B, Hkv, d = int(rs.integers(1, 5)), int(rs.choice([1, 4, 8])), 128
    q = int(rs.choice([32, 64, 96, 128]))
    C = 1000 + q
    t = C - q
    o = [int(v) for v in rs.integers(0, t - q + 1, size=B)]
    note(f"random round trip seed={seed} B={B} Hkv={Hkv} q={q} o={o}")
    Kc = torch.from_numpy(rs.standard_normal((B, C, Hkv, d)).astype(np.float32)).bfloat16().cuda()
    Vc = torch.from_numpy(rs.standard_normal((B, C, Hkv, d)).astype(np.float32)).bfloat16().cuda()
    K0, V0 = Kc.clone(), Vc.clone()
    o_t = torch.tensor(o, dtype=torch.int32).cuda()
    bd.kv_scatter(Kc, Vc, Kc, Vc, o_t, t, q)
    idx = torch.tensor([[[ob + j for j in range(q)]] * Hkv for ob in o], dtype=torch.int32).cuda()
    pk = torch.zeros((B, q, Hkv, d), dtype=torch.bfloat16, device="cuda")
    pv = torch.zeros_like(pk)
    bd.gather(Kc, Vc, idx, torch.full((B,), q, dtype=torch.int32).cuda(), pk, pv)
    torch.cuda.synchronize()
    assert np.array_equal(bits(pk), bits(K0[:, t:])) and np.array_equal(bits(pv), bits(V0[:, t:]))
    want_k = orc.kv_scatter(bits(K0)[None], bits(K0)[None], o, t, q)[0]
    assert np.array_equal(bits(Kc), want_k)
