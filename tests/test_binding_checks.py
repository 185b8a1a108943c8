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
