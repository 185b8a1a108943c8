"""Pins for the oracle's gather (HERALD Sec. IV-B3) and KV write-back
scatter (FlowBlock review Eq. (7) / paper Eq. 6)."""
import numpy as np

from oracle import bd_oracle as orc


def test_gather_vs_fancy_indexing():
    rs = np.random.default_rng(0)
    B, S, Hkv, d, kmax = 3, 40, 4, 8, 12
    src = rs.standard_normal((B, S, Hkv, d)).astype(np.float32)
    k_cnt = np.array([12, 5, 0])
    idx = np.full((B, Hkv, kmax), -1)
    for b in range(B):
        for h in range(Hkv):
            idx[b, h, :k_cnt[b]] = np.sort(rs.choice(S, k_cnt[b], replace=False))
    canary = np.full((B, kmax, Hkv, d), 123.5, np.float32)
    pool = orc.gather(src, idx, k_cnt, canary)
    for b in range(B):
        for h in range(Hkv):
            k = k_cnt[b]
            np.testing.assert_array_equal(pool[b, :k, h], src[b][idx[b, h, :k], h])
            assert (pool[b, k:, h] == 123.5).all()


def test_scatter_layers_alias_and_canaries():
    rs = np.random.default_rng(1)
    L, B, C, Hkv, d, q = 3, 4, 64, 2, 4, 8
    t = C - q
    data = rs.standard_normal((L, B, C, Hkv, d))
    o = np.array([0, 17, 40, t])            # o = t writes the tail onto itself
    out = orc.kv_scatter(data, data, o, t, q)
    for b in range(B):
        ob = o[b]
        np.testing.assert_array_equal(out[:, b, ob:ob + q], data[:, b, t:t + q])
        keep = np.ones(C, bool)
        keep[ob:ob + q] = False
        np.testing.assert_array_equal(out[:, b, keep], data[:, b, keep])


def test_scatter_then_gather_round_trip():
    rs = np.random.default_rng(2)
    B, C, Hkv, d, q = 2, 50, 3, 4, 6
    t = C - q
    cache = rs.standard_normal((1, B, C, Hkv, d))
    o = np.array([5, 30])
    after = orc.kv_scatter(cache, cache, o, t, q)[0]
    idx = np.stack([np.stack([o[b] + np.arange(q)] * Hkv) for b in range(B)])
    pool = orc.gather(after, idx, [q, q], np.zeros((B, q, Hkv, d)))
    np.testing.assert_array_equal(pool, cache[0, :, t:t + q])


def test_scatter_row_subset():
    rs = np.random.default_rng(3)
    B, C, Hkv, d, q = 3, 30, 1, 2, 4
    data = rs.standard_normal((1, B, C, Hkv, d))
    present = rs.standard_normal((1, B, C, Hkv, d))
    out = orc.kv_scatter(present, data, [1, 2, 3], C - q, q, rows=[1])
    np.testing.assert_array_equal(out[:, [0, 2]], data[:, [0, 2]])
    np.testing.assert_array_equal(out[0, 1, 2:6], present[0, 1, C - q:])
