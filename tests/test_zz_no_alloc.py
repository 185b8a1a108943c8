"""GPU check of bd_attn_packed_noalloc, the allocation-free variant of
bd_attn_packed: through the C-ABI, its outputs (O and LSE) must equal
bd_attn_packed's with a caller workspace bit for bit, on calls in a row
whose scratch needs differ (split-prefix partials, then a smaller split,
then the longest-first row order only), so stale scratch from an earlier
call never leaks into a later one."""
import pytest
import torch

import synth
from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


def _pool_case(B, P, seed):
    """B rows over a pool of P entries each (HERALD's denoising attention),
    one 32-query block, 32/8 heads."""
    g = torch.Generator().manual_seed(seed)
    Hq, Hkv, d, q = 32, 8, 128, 32
    s = d ** -0.5
    mk = lambda *shape: (torch.randn(shape, generator=g) * s).bfloat16().cuda()
    Q, pk, pv = mk(B, q, Hq, d), mk(B, P, Hkv, d), mk(B, P, Hkv, d)
    wk, wv = mk(B, q, Hkv, d), mk(B, q, Hkv, d)
    p_len = torch.tensor([P - 37 * (b % 3) for b in range(B)], dtype=torch.int32).cuda()
    return Q, pk, pv, p_len, P, wk, wv, 32, s


def _cache_case(seed):
    """Many rows over their own cache (the serving mix's dense launch shape,
    reduced): the plan orders the rows longest first."""
    wl = synth.serving_mix(seed=seed, B=40, p_lo=300, p_hi=3000, W=4, sparse_above=10 ** 9)
    Kc, Vc, Q, o = wl.Kc.cuda(), wl.Vc.cuda(), wl.Q.cuda(), wl.o.cuda()
    t = wl.t
    return Q, Kc, Vc, o, int(wl.o.max()), Kc[:, t:], Vc[:, t:], wl.bl, wl.sm_scale


def _compare(bd, case, label):
    Q, pk, pv, p_len, p_max, wk, wv, bl, scale = case
    B, q, Hq, d = Q.shape
    Hkv = pk.shape[2]
    need = bd.attn_workspace_size(Q.dtype, B, Hq, Hkv, d, q, B, p_max)
    assert 0 < need <= bd.noalloc_scratch_bytes(), (label, need)
    note(f"noalloc {label}: B={B} p_max={p_max} scratch={need} bytes")
    out_ref = torch.full_like(Q, float("nan"))
    lse_ref = torch.full((B, Hq, q), float("nan"), device="cuda")
    bd.attn_packed(Q, pk, pv, p_len, p_max, wk, wv, bl, scale, out=out_ref, lse=lse_ref)
    out = torch.full_like(Q, float("nan"))
    lse = torch.full((B, Hq, q), float("nan"), device="cuda")
    bd.attn_packed_noalloc(Q, pk, pv, p_len, p_max, wk, wv, bl, scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out_ref.float()).all() and torch.isfinite(lse_ref).all(), label
    assert torch.equal(out, out_ref), f"{label}: outputs differ"
    assert torch.equal(lse, lse_ref), f"{label}: LSE differs"


def test_noalloc_matches_workspace_calls(bd):
    # 1: 4 rows x 8 KV heads over 1638-entry pools: the prefix is split and
    #    the partials fill most of the scratch
    _compare(bd, _pool_case(4, 1638, 0), "pool 4x1638")
    # 2: a smaller split right after it (fewer units, shorter chunks)
    _compare(bd, _pool_case(2, 700, 1), "pool 2x700")
    # 3: 40 rows over their own caches: no split, the row order only
    _compare(bd, _cache_case(2), "cache 40 rows")
    # 4: the first shape again after the others
    _compare(bd, _pool_case(4, 1638, 3), "pool 4x1638 again")
