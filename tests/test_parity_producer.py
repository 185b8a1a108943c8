"""GPU parity of bd_qkv_rope_write (Flash-dLLM's fused Flash-Cache producer:
QKV projection + absolute-position RoPE + cache write) against the float64
oracle's qkv_rope.

Outputs within the bf16 bound |g - r| <= 2e-2 + 1e-2 |r| and a per-(row,
head) normalised error <= 1e-2; cache rows outside the written window and
positions past the capacity are compared bit-exactly with their old values.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import note
from oracle import bd_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


def _check(g, r, label):
    g = g.detach().cpu().double().numpy()
    assert np.isfinite(g).all(), label
    err = np.abs(g - r)
    bad = err > 2e-2 + 1e-2 * np.abs(r)
    assert not bad.any(), f"{label}: {bad.sum()} out of tolerance, max err {err.max():.3e}"
    num = np.sqrt(((g - r) ** 2).sum(axis=(-3, -1)))
    den = np.sqrt((r ** 2).sum(axis=(-3, -1)))
    assert (num / den).max() <= 1e-2, f"{label}: normalised error {(num / den).max():.3e}"


def _case(seed, B, q, Dm, Hq, Hkv, d=128):
    rs = np.random.default_rng(seed)
    X = torch.from_numpy(rs.standard_normal((B, q, Dm)).astype(np.float32)).bfloat16()
    W = torch.from_numpy((rs.standard_normal(((Hq + 2 * Hkv) * d, Dm)) / math.sqrt(Dm))
                         .astype(np.float32)).bfloat16()
    return X, W


def _run(bd, X, W, rope_pos, dst_pos, Hq, Hkv, C, base=10000.0):
    B, q, Dm = X.shape
    d = 128
    Kc = torch.full((B, C, Hkv, d), 7.0, dtype=torch.bfloat16, device="cuda")
    Vc = torch.full((B, C, Hkv, d), -7.0, dtype=torch.bfloat16, device="cuda")
    Qo = torch.full((B, q, Hq, d), 9.0, dtype=torch.bfloat16, device="cuda")
    i32 = lambda v: torch.tensor(v, dtype=torch.int32).cuda()
    bd.qkv_rope_write(X.cuda(), W.cuda(), i32(rope_pos), Hq, Hkv, Qo, Kc, Vc, i32(dst_pos), base)
    torch.cuda.synchronize()
    return Qo, Kc, Vc


@pytest.mark.parametrize("B,q,Dm,Hq,Hkv,rope_pos", [
    (3, 40, 256, 8, 2, [0, 1000, 131000]),      # one ragged token tile, large positions
    (2, 256, 320, 5, 1, [3, 70000]),            # odd hidden-tile count, odd head count, XCD block order
    (3, 300, 256, 8, 2, [11, 0, 90000]),        # ragged group of head pairs, 24 blocks in XCD order
    (2, 200, 512, 4, 4, [17, 4096]),            # tiles spanning rows
    (5, 64, 128, 16, 2, [5, 9, 33, 70000, 1]),  # G = 8
    (3, 40, 128, 1, 1, [2, 50, 7]),             # three heads: an odd head count
    (2, 128, 256, 4, 2, [1000003, 2500000]),   # stepped rotation at positions past 1e6
    (2, 96, 64, 4, 2, [5, 77]),                 # one hidden tile (no loop iteration after the first)
    (1, 64, 192, 2, 1, [0]),                    # three hidden tiles, one token quarter per wave row
])
def test_producer_small(bd, B, q, Dm, Hq, Hkv, rope_pos):
    note(f"producer B={B} q={q} Dm={Dm} Hq={Hq} Hkv={Hkv}")
    X, W = _case(B * q + Dm, B, q, Dm, Hq, Hkv)
    C = q + 300
    dst = [(b * 37) % 250 for b in range(B)]
    Qo, Kc, Vc = _run(bd, X, W, rope_pos, dst, Hq, Hkv, C)
    Q, K, V = orc.qkv_rope(X, W, rope_pos, Hq, Hkv)
    _check(Qo, Q, "q")
    Kg, Vg = Kc.cpu(), Vc.cpu()
    for b in range(B):
        _check(Kg[b:b + 1, dst[b]:dst[b] + q], K[b:b + 1], f"k row {b}")
        _check(Vg[b:b + 1, dst[b]:dst[b] + q], V[b:b + 1], f"v row {b}")
        keep = np.ones(C, bool)
        keep[dst[b]:dst[b] + q] = False
        assert (Kg[b, keep] == 7.0).all() and (Vg[b, keep] == -7.0).all(), "write outside the window"


def test_producer_capacity_edge(bd):
    """Window positions at or past the cache capacity are not written."""
    note("producer capacity edge")
    B, q, Dm, Hq, Hkv = 2, 64, 128, 4, 2
    X, W = _case(5, B, q, Dm, Hq, Hkv)
    C = 100
    dst = [C - 10, 0]
    Qo, Kc, Vc = _run(bd, X, W, [3, 3], dst, Hq, Hkv, C)
    Q, K, V = orc.qkv_rope(X, W, [3, 3], Hq, Hkv)
    _check(Qo, Q, "q")
    _check(Kc[0:1, C - 10:].cpu(), K[0:1, :10], "k tail")
    _check(Vc[1:2, :q].cpu(), V[1:2], "v row 1")
    assert (Kc[0, :C - 10].cpu() == 7.0).all()


def test_producer_serving_mix_shape(bd):
    """The serving-mix shape the bench times (64 rows x 128 window tokens,
    hidden 4096, 32/8 heads, keys and values written at the window tail):
    two sampled rows against the oracle; every output finite."""
    note("producer serving-mix shape")
    B, q, Dm, Hq, Hkv = 64, 128, 4096, 32, 8
    X, W = _case(11, B, q, Dm, Hq, Hkv)
    rs = np.random.default_rng(12)
    rope_pos = [int(v) for v in rs.integers(1024, 16384, size=B)]
    C = 16384 + 2 * q
    t = C - q
    Qo, Kc, Vc = _run(bd, X, W, rope_pos, [t] * B, Hq, Hkv, C)
    assert torch.isfinite(Qo).all()
    for b in (0, 41):
        Q, K, V = orc.qkv_rope(X[b:b + 1], W, rope_pos[b:b + 1], Hq, Hkv)
        _check(Qo[b:b + 1], Q, f"q row {b}")
        _check(Kc[b:b + 1, t:].cpu(), K, f"k row {b}")
        _check(Vc[b:b + 1, t:].cpu(), V, f"v row {b}")


def test_producer_strided_hidden_states(bd):
    """Hidden states as a view into a larger buffer (row and token strides
    that are not q * Dm and Dm): the tile transfers address x through its
    strides, tokens of a ragged last tile re-read the last token."""
    note("producer strided x")
    B, q, Dm, Hq, Hkv = 3, 72, 192, 4, 2
    rs = np.random.default_rng(31)
    big = torch.from_numpy(rs.standard_normal((B, q + 9, Dm + 64)).astype(np.float32)).bfloat16()
    X = big[:, 5:5 + q, 32:32 + Dm]                     # strides (81 * 256, 256, 1)
    _, W = _case(32, B, q, Dm, Hq, Hkv)
    rope_pos = [4, 1900, 70001]
    dst = [0, 13, 40]
    C = q + 64
    Kc = torch.full((B, C, Hkv, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    Vc = torch.full((B, C, Hkv, 128), -7.0, dtype=torch.bfloat16, device="cuda")
    Qo = torch.empty((B, q, Hq, 128), dtype=torch.bfloat16, device="cuda")
    i32 = lambda v: torch.tensor(v, dtype=torch.int32).cuda()
    Xg = big.cuda()[:, 5:5 + q, 32:32 + Dm]
    assert not Xg.is_contiguous()
    bd.qkv_rope_write(Xg, W.cuda(), i32(rope_pos), Hq, Hkv, Qo, Kc, Vc, i32(dst))
    torch.cuda.synchronize()
    Q, K, V = orc.qkv_rope(X.contiguous(), W, rope_pos, Hq, Hkv)
    _check(Qo, Q, "q (strided x)")
    for b in range(B):
        _check(Kc.cpu()[b:b + 1, dst[b]:dst[b] + q], K[b:b + 1], f"k row {b} (strided x)")
        _check(Vc.cpu()[b:b + 1, dst[b]:dst[b] + q], V[b:b + 1], f"v row {b} (strided x)")
