"""Pins for the oracle's fused producer (Flash-dLLM's Flash-Cache: QKV
projection, RoPE, cache write) and its rotary embedding (HERALD Eq. (1)).
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import bd_oracle as orc


def test_rope_position_zero_is_identity_and_norms_kept():
    rs = np.random.default_rng(1)
    x = rs.standard_normal((5, 16))
    np.testing.assert_array_equal(orc.rope(x, np.zeros(5)), x)
    y = orc.rope(x, np.arange(5) * 997)
    # every (j, j + d/2) pair is rotated, so its norm is kept
    np.testing.assert_allclose(x[:, :8] ** 2 + x[:, 8:] ** 2, y[:, :8] ** 2 + y[:, 8:] ** 2, rtol=1e-12)


def test_rope_relative_offset_eq1():
    """HERALD Eq. (1): the score of a rotated query at p and a rotated key at
    s depends only on p - s."""
    rs = np.random.default_rng(2)
    qv, kv = rs.standard_normal(32), rs.standard_normal(32)
    base = []
    for p, s in ((40, 7), (1033, 1000), (33, 0), (90033, 90000)):
        sc = orc.rope(qv[None], [p])[0] @ orc.rope(kv[None], [s])[0]
        base.append(sc)
    np.testing.assert_allclose(base, base[0], rtol=1e-9)


def test_rope_as_complex_rotation():
    """The same map written as complex multiplication of (x_j + i x_{j+d/2})
    by exp(i p theta_j), theta_j = 10000^(-2j/d)."""
    rs = np.random.default_rng(3)
    d = 128
    x = rs.standard_normal((7, d))
    pos = np.array([0, 1, 5, 100, 4095, 16384, 131071])
    z = (x[:, :d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, None] *
                                                      10000.0 ** (-np.arange(d // 2) * 2 / d))
    np.testing.assert_allclose(orc.rope(x, pos), np.concatenate([z.real, z.imag], 1), rtol=1e-12,
                               atol=1e-12)


def test_qkv_rope_vs_linear_and_positions():
    """Projection = torch linear in float64; queries and keys rotated at
    rope_pos[b] + i, values not rotated; head order q, k, v."""
    rs = np.random.default_rng(4)
    B, q, Dm, Hq, Hkv, d = 2, 6, 24, 4, 2, 8
    X = rs.standard_normal((B, q, Dm))
    W = rs.standard_normal(((Hq + 2 * Hkv) * d, Dm))
    pos0 = np.array([0, 1000])
    Q, K, V = orc.qkv_rope(X, W, pos0, Hq, Hkv)
    Y = F.linear(torch.from_numpy(X), torch.from_numpy(W)).numpy().reshape(B, q, Hq + 2 * Hkv, d)
    for b in range(B):
        pos = pos0[b] + np.arange(q)
        for hq in range(Hq):
            np.testing.assert_allclose(Q[b, :, hq], orc.rope(Y[b, :, hq], pos), rtol=1e-12, atol=1e-12)
        for h in range(Hkv):
            np.testing.assert_allclose(K[b, :, h], orc.rope(Y[b, :, Hq + h], pos), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(V[b, :, h], Y[b, :, Hq + Hkv + h], rtol=1e-12, atol=1e-12)
    # row 0 starts at position 0: its first token is the plain projection
    np.testing.assert_allclose(Q[0, 0], Y[0, 0, :Hq], rtol=1e-12, atol=1e-12)
    # shifting every position leaves query-key scores unchanged (Eq. (1))
    Q2, K2, _ = orc.qkv_rope(X, W, pos0 + 12345, Hq, Hkv)
    s1 = np.einsum("bihd,bjhd->bhij", Q[:, :, :Hkv], K)
    s2 = np.einsum("bihd,bjhd->bhij", Q2[:, :, :Hkv], K2)
    np.testing.assert_allclose(s1, s2, rtol=1e-8, atol=1e-8)
