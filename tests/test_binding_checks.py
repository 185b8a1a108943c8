"""The binding refuses output and per-row buffers whose shape, dtype or
layout differs from what the C-ABI indexes (a wrong shape raises on the host
instead of writing out of bounds on the GPU).  Nothing here launches a kernel
with a bad buffer."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


def test_select_buffers(bd):
    B, C, Hq, Hkv, d = 2, 300, 8, 2, 128
    q = torch.zeros((B, 4, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, C, Hkv, d), dtype=torch.bfloat16, device="cuda")
    i32 = lambda *v: torch.tensor(v, dtype=torch.int32, device="cuda")
    for fn in (bd.select, bd.select_multi):
        with pytest.raises(ValueError, match="idx_out"):
            fn(q, k, i32(100, 50), 100, i32(5, 5), 5, 0.1,
               idx_out=torch.empty((B, Hkv, 4), dtype=torch.int32, device="cuda"))
        with pytest.raises(ValueError, match="score_out"):
            fn(q, k, i32(100, 50), 100, i32(5, 5), 5, 0.1,
               score_out=torch.empty((B, Hkv, 99), device="cuda"))
        with pytest.raises(ValueError, match="s_len"):
            fn(q, k, i32(100), 100, i32(5, 5), 5, 0.1)


def test_attention_and_move_buffers(bd):
    B, C, Hq, Hkv, d, q = 2, 300, 8, 2, 128, 64
    Q = torch.zeros((B, q, Hq, d), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((B, C, Hkv, d), dtype=torch.bfloat16, device="cuda")
    t = C - q
    i32 = lambda *v: torch.tensor(v, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="lse"):
        bd.attn_packed(Q, K, K, i32(10, 20), 20, K[:, t:], K[:, t:], 32, 0.1,
                       lse=torch.empty((B, Hq, q - 1), device="cuda"))
    with pytest.raises(ValueError, match="out"):
        bd.attn_packed(Q, K, K, i32(10, 20), 20, K[:, t:], K[:, t:], 32, 0.1,
                       out=torch.empty((B, q, Hq, d), device="cuda"))
    with pytest.raises(ValueError, match="p_len"):
        bd.attn_packed(Q, K, K, i32(10), 20, K[:, t:], K[:, t:], 32, 0.1)
    with pytest.raises(ValueError, match="o must hold"):
        bd.kv_scatter(K, K, K, K, i32(3), t, q)
    with pytest.raises(ValueError, match="idx"):
        bd.gather(K, K, torch.zeros((B, Hkv + 1, 4), dtype=torch.int32, device="cuda"), i32(4, 4),
                  torch.zeros((B, 4, Hkv, d), dtype=torch.bfloat16, device="cuda"),
                  torch.zeros((B, 4, Hkv, d), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="o must hold"):
        bd.mask_materialize(3, C, q, 32, i32(0, 1))


def test_producer_buffers(bd):
    B, q, Dm, Hq, Hkv, d, C = 2, 16, 128, 4, 2, 128, 64
    x = torch.zeros((B, q, Dm), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(((Hq + 2 * Hkv) * d, Dm), dtype=torch.bfloat16, device="cuda")
    qo = torch.zeros((B, q, Hq, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, C, Hkv, d), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="w must be"):
        bd.qkv_rope_write(x, w[:-1], pos, Hq, Hkv, qo, kc, kc.clone(), pos)
    with pytest.raises(ValueError, match="q_out"):
        bd.qkv_rope_write(x, w, pos, Hq, Hkv, qo[:, :-1], kc, kc.clone(), pos)
    with pytest.raises(ValueError, match="k_cache"):
        bd.qkv_rope_write(x, w, pos, Hq, Hkv, qo, kc[:, :, :1], kc[:, :, :1].clone(), pos)
    with pytest.raises(ValueError, match="dst_pos"):
        bd.qkv_rope_write(x, w, pos, Hq, Hkv, qo, kc, kc.clone(), pos[:1])


def test_source_and_target_tensors_checked(bd):
    """Every tensor the C-ABI indexes with its own strides (gather pools,
    scatter targets, attention prefix and window sources, the selection's K,
    the producer's outputs) must match the dtype, heads and head dim of the
    tensor its strides are taken from; otherwise the call raises on the host
    before any launch."""
    B, C, Hq, Hkv, d, q = 2, 300, 8, 2, 128, 64
    bf, f32 = torch.bfloat16, torch.float32
    z = lambda shape, dt=bf: torch.zeros(shape, dtype=dt, device="cuda")
    i32 = lambda *v: torch.tensor(v, dtype=torch.int32, device="cuda")
    K, Kf = z((B, C, Hkv, d)), z((B, C, Hkv, d), f32)
    idx = torch.zeros((B, Hkv, 4), dtype=torch.int32, device="cuda")
    # gather: pool dtype, rows, heads, capacity; V pool shape
    for bad, msg in ((z((B, 4, Hkv, d), f32), "k_pool must be"), (z((B - 1, 4, Hkv, d)), "k_pool must be"),
                     (z((B, 4, Hkv + 1, d)), "k_pool must be"), (z((B, 3, Hkv, d)), "k_pool must be")):
        with pytest.raises(ValueError, match=msg):
            bd.gather(K, K, idx, i32(4, 4), bad, bad)
    with pytest.raises(ValueError, match="k_pool and v_pool"):
        bd.gather(K, K, idx, i32(4, 4), z((B, 4, Hkv, d)), z((B, 5, Hkv, d)))
    with pytest.raises(ValueError, match="k_src and v_src"):
        bd.gather(K, K[:, :-1], idx, i32(4, 4), z((B, 4, Hkv, d)), z((B, 4, Hkv, d)))
    with pytest.raises(ValueError, match="k_pool must be"):
        bd.gather(Kf, Kf, idx, i32(4, 4), z((B, 4, Hkv, d)), z((B, 4, Hkv, d)))
    # scatter: target dtype, rows, heads; V target shape
    t = C - q
    for bad in (z((B, C, Hkv, d), f32), z((B - 1, C, Hkv, d)), z((B, C, Hkv, d // 2))):
        with pytest.raises(ValueError, match="data_k must be"):
            bd.kv_scatter(K, K, bad, bad, i32(0, 0), t, q)
    with pytest.raises(ValueError, match="data_k and data_v"):
        bd.kv_scatter(K, K, z((B, C, Hkv, d)), z((B, C - 1, Hkv, d)), i32(0, 0), t, q)
    with pytest.raises(ValueError, match="both be given"):
        bd.kv_scatter(K, K, z((B, C, Hkv, d)), None, i32(0, 0), t, q)
    # attention: prefix and window dtype, heads, rows; window length
    Q, Qf = z((B, q, Hq, d)), z((B, q, Hq, d), f32)
    with pytest.raises(ValueError, match="pk must be"):
        bd.attn_packed(Qf, K, K, i32(10, 20), 20, Kf[:, t:], Kf[:, t:], 32, 0.1)
    with pytest.raises(ValueError, match="pv must be"):
        bd.attn_packed(Q, K, Kf, i32(10, 20), 20, K[:, t:], K[:, t:], 32, 0.1)
    with pytest.raises(ValueError, match="wk must be"):
        bd.attn_packed(Q, K, K, i32(10, 20), 20, K[:, t + 1:], K[:, t + 1:], 32, 0.1)
    with pytest.raises(ValueError, match="pk must be"):
        bd.attn_packed(Q, K[:1], K[:1], i32(10, 20), 20, K[:, t:], K[:, t:], 32, 0.1)
    with pytest.raises(ValueError, match="pk_b must be"):
        bd.attn_packed_dual(Q, (i32(0), K, K, i32(10, 20), 20), (i32(1), Kf, Kf, i32(4, 4), 4),
                            K[:, t:], K[:, t:], 32, 0.1)
    with pytest.raises(ValueError, match="pk_a and pv_a"):
        bd.attn_packed_dual(Q, (i32(0), K, K[:, :-1], i32(10, 20), 20), (i32(1), K, K, i32(4, 4), 4),
                            K[:, t:], K[:, t:], 32, 0.1)
    # selection: K dtype and head dim
    for fn in (bd.select, bd.select_multi):
        with pytest.raises(ValueError, match="k must be"):
            fn(z((B, 4, Hq, d)), Kf, i32(100, 50), 100, i32(5, 5), 5, 0.1)
    # producer outputs share x's dtype
    x = z((B, 16, 128))
    w = z(((Hq + 2 * Hkv) * d, 128))
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="q_out must be"):
        bd.qkv_rope_write(x, w, pos, Hq, Hkv, z((B, 16, Hq, d), f32), K, K.clone(), pos)
    with pytest.raises(ValueError, match="k_cache must be"):
        bd.qkv_rope_write(x, w, pos, Hq, Hkv, z((B, 16, Hq, d)), Kf, Kf.clone(), pos)
