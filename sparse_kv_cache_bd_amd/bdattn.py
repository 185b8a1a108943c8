"""Thin ctypes binding of libbdattn (argument marshalling only).

Every function takes torch tensors on the GPU, turns them into device
pointers, element strides and the current HIP stream, and calls the C-ABI
entry point of the same name.  All computation happens in the HIP kernels;
there is no CPU path.  A missing library or a CPU tensor raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbdattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "bdattn.h")

BD_OK, BD_ERR_INVALID_ARG, BD_ERR_UNSUPPORTED, BD_ERR_HIP, BD_ERR_WORKSPACE = 0, 1, 2, 3, 4
BD_BF16, BD_F32 = 0, 1
BD_REP_MEAN, BD_REP_ROW = 0, 1
BD_MASK_BLOCK_CAUSAL, BD_MASK_ISOLATED, BD_MASK_SHARED_FIRST = 0, 1, 2
# device check mode: status bits (bd_check_*)
CHECK_BITS = {"row": 0x01, "length": 0x02, "offset": 0x04, "alias": 0x08, "index": 0x10,
              "page": 0x20, "queries": 0x40}
MASK_MODES = {"block_causal": BD_MASK_BLOCK_CAUSAL, "isolated": BD_MASK_ISOLATED,
              "shared_first": BD_MASK_SHARED_FIRST}

_DTYPE = {torch.bfloat16: BD_BF16, torch.float32: BD_F32}

_c_i64_2 = ctypes.c_int64 * 2
_c_i64_3 = ctypes.c_int64 * 3
_c_i64_4 = ctypes.c_int64 * 4
_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

_SIGS = {
    "bd_version": (ctypes.c_char_p, []),
    "bd_last_error": (ctypes.c_char_p, []),
    "bd_kv_scatter": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _i,
                           _vp, _vp, _i, _vp]),
    "bd_gather": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _vp, _i, _vp]),
    "bd_select_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "bd_select": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _i, _i, _i, _vp, _vp, _i, _vp, _i, _vp, _i,
                       ctypes.c_float, _vp, _vp, _vp, _sz, _vp]),
    "bd_select_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "bd_select_attn": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp,
                            _i, _vp, _i, ctypes.c_float, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bd_select_multi_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "bd_select_multi": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp, _i, _vp, _i, _vp, _i,
                             ctypes.c_float, _vp, _vp, _vp, _sz, _vp]),
    "bd_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "bd_attn_packed": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _i,
                            _vp, _i, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _sz,
                            _vp]),
    "bd_attn_dual_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "bd_attn_packed_dual": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                 _vp, _i, _vp, _vp, _vp, _i, _vp, _i,
                                 _vp, _i, _vp, _vp, _vp, _i, _vp, _i,
                                 _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bd_attn_packed_noalloc": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp,
                                    _i, _vp, _i, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                                    _vp]),
    "bd_attn_block_table_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "bd_attn_block_table": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp, _i, _vp, _i, _vp, _vp, _vp, _i,
                                 _i, _i, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                                 _vp, _sz, _vp]),
    "bd_attn_packed_masked": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _vp, _i, _vp, _vp, _vp, _vp,
                                   _vp, _i, _vp, _i, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                                   _vp, _sz, _vp]),
    "bd_mask_materialize": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "bd_check_attn": (_i, [_i, _vp, _i, _vp, _i, _i, _i, _vp, _vp]),
    "bd_check_scatter": (_i, [_i, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp]),
    "bd_check_gather": (_i, [_i, _i, _vp, _i, _vp, _i, _vp, _vp]),
    "bd_check_select": (_i, [_i, _vp, _i, _i, _vp, _i, _vp, _vp]),
    "bd_check_block_table": (_i, [_i, _i, _vp, _i, _vp, _i, _i, _i, _i, _vp, _vp]),
    "bd_qkv_rope_write": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, ctypes.c_float,
                               _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp]),
}

_lib = None


class BdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libbdattn error {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libbdattn.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def noalloc_scratch_bytes() -> int:
    """BD_NOALLOC_SCRATCH_BYTES as the public header defines it."""
    with open(HEADER_PATH) as f:
        m = re.search(r"#define\s+BD_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", f.read())
    return int(m.group(1)) << int(m.group(2))


def header_functions() -> list[str]:
    """Names of the functions the public header declares."""
    with open(HEADER_PATH) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(bd_[a-z_0-9]+)\s*\(", txt)))


def version() -> str:
    return lib().bd_version().decode()


def last_error() -> str:
    return lib().bd_last_error().decode()


def _check(code: int):
    if code != BD_OK:
        raise BdError(code, last_error())


def _dev(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor on the GPU")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _strides(t: torch.Tensor, n: int):
    if t.stride(-1) != 1:
        raise ValueError("the head dimension must be contiguous")
    st = list(t.stride()[:-1])
    assert len(st) == n, (t.shape, n)
    return {2: _c_i64_2, 3: _c_i64_3, 4: _c_i64_4}[n](*st)


def _i32(t, name):
    t = _dev(t, name)
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    return t


def _buf(t, name, shape, dtype):
    """An output or per-row buffer the C-ABI indexes as contiguous memory:
    checked here so that a wrong shape raises instead of writing out of
    bounds on the GPU."""
    if t is None:
        return None
    t = _dev(t, name)
    if t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")
    return t


def _rows(t, name, B):
    t = _i32(t, name)
    if t.numel() < B:
        raise ValueError(f"{name} must hold at least {B} entries")
    return t


def _kv(t, name, B, Hkv, d, dtype, min_len=0, lead=()):
    """A K/V-like tensor ``[*lead, >= B, >= min_len, Hkv, d]`` the C-ABI
    indexes with its own strides: dtype, rank, row count, head count and
    head dim are checked here, so a mismatched buffer raises instead of
    being read or written out of bounds."""
    t = _dev(t, name)
    n = len(lead) + 4
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    sh = tuple(t.shape)
    if sh[:len(lead)] != tuple(lead) or sh[len(lead)] < B or sh[len(lead) + 1] < min_len or \
            sh[len(lead) + 2:] != (Hkv, d):
        want = ", ".join([*map(str, lead), f">={B}", f">={min_len}", str(Hkv), str(d)])
        raise ValueError(f"{name} must be [{want}], got {sh}")
    return t


def _pair(k, v, kname, vname):
    """K and V of one source share shape and strides (one stride set crosses
    the C-ABI for both)."""
    if v is not None and (v.shape != k.shape or v.stride() != k.stride()):
        raise ValueError(f"{kname} and {vname} must share shape and strides")


def workspace(nbytes: int, device=None) -> torch.Tensor | None:
    """Caller-owned workspace (256-byte aligned: torch allocations are)."""
    if nbytes <= 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")


# ---------------------------------------------------------------------------

def kv_scatter(present_k, present_v, data_k, data_v, o, t: int, q: int, row_ids=None):
    """Eq. (7) write-back.  present_*/data_*: [L, B, P, Hkv, d] or [B, P, Hkv, d]."""
    pk, dk = _dev(present_k, "present_k"), _dev(data_k, "data_k")
    pv, dv = _dev(present_v, "present_v"), _dev(data_v, "data_v")
    if (pv is None) != (dv is None):
        raise ValueError("present_v and data_v must both be given or both be None")
    if pk.dim() == 4:
        pk, dk = pk.unsqueeze(0), dk.unsqueeze(0)
        pv = pv.unsqueeze(0) if pv is not None else None
        dv = dv.unsqueeze(0) if dv is not None else None
    if pk.dim() != 5:
        raise ValueError("present_k must be [L, B, P, Hkv, d] or [B, P, Hkv, d]")
    L, B, Pcap, Hkv, d = pk.shape
    dk = _kv(dk, "data_k", B, Hkv, d, pk.dtype, lead=(L,))
    _pair(pk, pv, "present_k", "present_v")
    _pair(dk, dv, "data_k", "data_v")
    o = _rows(o, "o", B)
    rid = _i32(row_ids, "row_ids") if row_ids is not None else None
    n_rows = B if rid is None else rid.numel()
    _check(lib().bd_kv_scatter(_DTYPE[pk.dtype], B, Hkv, d, q, L, _ptr(pk), _ptr(pv),
                               _strides(pk, 4), Pcap, t, _ptr(dk), _ptr(dv), _strides(dk, 4),
                               dk.shape[2], _ptr(o), _ptr(rid), n_rows, _stream()))


def gather(k_src, v_src, idx, k_cnt, k_pool, v_pool):
    """Pool gather.  *_src: [B, S, Hkv, d]; idx [B, Hkv, k_max]; pools [B, >=k_max, Hkv, d]."""
    ks, kp = _dev(k_src, "k_src"), _dev(k_pool, "k_pool")
    vs, vp = _dev(v_src, "v_src"), _dev(v_pool, "v_pool")
    if (vs is None) != (vp is None):
        raise ValueError("v_src and v_pool must both be given or both be None")
    if ks.dim() != 4:
        raise ValueError("k_src must be [B, S, Hkv, d]")
    B, S, Hkv, d = ks.shape
    idx = _i32(idx, "idx")
    if idx.dim() != 3 or tuple(idx.shape[:2]) != (B, Hkv):
        raise ValueError(f"idx must be [{B}, {Hkv}, k_max]")
    k_max = idx.shape[2]
    kp = _kv(kp, "k_pool", B, Hkv, d, ks.dtype, min_len=k_max)
    _pair(ks, vs, "k_src", "v_src")
    _pair(kp, vp, "k_pool", "v_pool")
    k_cnt = _rows(k_cnt, "k_cnt", B)
    _check(lib().bd_gather(_DTYPE[ks.dtype], B, Hkv, d, _ptr(ks), _ptr(vs), _strides(ks, 3), S,
                           _ptr(idx), k_max, _ptr(k_cnt), _ptr(kp), _ptr(vp), _strides(kp, 3),
                           kp.shape[1], _stream()))


def select_workspace_size(B, Hq, Hkv, d, s_max, k_max) -> int:
    return int(lib().bd_select_workspace_size(B, Hq, Hkv, d, s_max, k_max))


def select(q, k, s_len, s_max: int, k_sel, k_max: int, sm_scale: float, rep_mode: int = BD_REP_MEAN,
           rep_row: int = 0, idx_out=None, score_out=None, ws=None):
    """Representative-query top-k.  q [B, nq, Hq, d]; k [B, C, Hkv, d].  Returns idx [B, Hkv, k_max]."""
    q, k = _dev(q, "q"), _dev(k, "k")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, nq, Hq, d] and k [B, C, Hkv, d]")
    B, nq, Hq, d = q.shape
    Hkv = k.shape[2]
    k = _kv(k, "k", B, Hkv, d, q.dtype)
    s_len, k_sel = _rows(s_len, "s_len", B), _rows(k_sel, "k_sel", B)
    if idx_out is None:
        idx_out = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=q.device)
    idx_out = _buf(idx_out, "idx_out", (B, Hkv, k_max), torch.int32)
    score_out = _buf(score_out, "score_out", (B, Hkv, s_max), torch.float32)
    need = select_workspace_size(B, Hq, Hkv, d, s_max, k_max)
    if ws is None:
        ws = workspace(need, q.device)
    _check(lib().bd_select(_DTYPE[q.dtype], B, Hq, Hkv, d, _ptr(q), _strides(q, 3), nq, rep_mode,
                           rep_row, _ptr(k), _strides(k, 3), k.shape[1], _ptr(s_len), s_max,
                           _ptr(k_sel), k_max, float(sm_scale), _ptr(idx_out), _ptr(score_out),
                           _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return idx_out


def select_attn_workspace_size(B, Hq, Hkv, d, s_max, k_max) -> int:
    return int(lib().bd_select_attn_workspace_size(B, Hq, Hkv, d, s_max, k_max))


def select_attn(q, k, v, s_len, s_max: int, k_sel, k_max: int, sm_scale: float,
                rep_mode: int = BD_REP_MEAN, rep_row: int = 0, idx_out=None, score_out=None,
                o_rep=None, ws=None):
    """Representative-query top-k plus the representative query's attention
    output.  q [B, nq, Hq, d]; k, v [B, C, Hkv, d].  Returns (idx [B, Hkv,
    k_max], o_rep [B, Hq, d])."""
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, nq, Hq, d] and k [B, C, Hkv, d]")
    B, nq, Hq, d = q.shape
    Hkv = k.shape[2]
    k = _kv(k, "k", B, Hkv, d, q.dtype)
    v = _kv(v, "v", B, Hkv, d, q.dtype, min_len=k.shape[1])
    s_len, k_sel = _rows(s_len, "s_len", B), _rows(k_sel, "k_sel", B)
    if idx_out is None:
        idx_out = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=q.device)
    idx_out = _buf(idx_out, "idx_out", (B, Hkv, k_max), torch.int32)
    score_out = _buf(score_out, "score_out", (B, Hkv, s_max), torch.float32)
    if o_rep is None:
        o_rep = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    o_rep = _buf(o_rep, "o_rep", (B, Hq, d), q.dtype)
    need = select_attn_workspace_size(B, Hq, Hkv, d, s_max, k_max)
    if ws is None:
        ws = workspace(need, q.device)
    _check(lib().bd_select_attn(_DTYPE[q.dtype], B, Hq, Hkv, d, _ptr(q), _strides(q, 3), nq,
                                rep_mode, rep_row, _ptr(k), _strides(k, 3), _ptr(v), _strides(v, 3),
                                k.shape[1], _ptr(s_len), s_max, _ptr(k_sel), k_max,
                                float(sm_scale), _ptr(idx_out), _ptr(score_out), _ptr(o_rep),
                                _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return idx_out, o_rep


def select_multi_workspace_size(B, Hq, Hkv, d, nq, s_max, k_max) -> int:
    return int(lib().bd_select_multi_workspace_size(B, Hq, Hkv, d, nq, s_max, k_max))


def select_multi(q, k, s_len, s_max: int, k_sel, k_max: int, sm_scale: float, idx_out=None,
                 score_out=None, ws=None):
    """Exact multi-query top-k: every one of the nq queries of q
    [B, nq, Hq, d] ranks k [B, C, Hkv, d].  Returns idx [B, Hkv, k_max]."""
    q, k = _dev(q, "q"), _dev(k, "k")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, nq, Hq, d] and k [B, C, Hkv, d]")
    B, nq, Hq, d = q.shape
    Hkv = k.shape[2]
    k = _kv(k, "k", B, Hkv, d, q.dtype)
    s_len, k_sel = _rows(s_len, "s_len", B), _rows(k_sel, "k_sel", B)
    if idx_out is None:
        idx_out = torch.empty((B, Hkv, k_max), dtype=torch.int32, device=q.device)
    idx_out = _buf(idx_out, "idx_out", (B, Hkv, k_max), torch.int32)
    score_out = _buf(score_out, "score_out", (B, Hkv, s_max), torch.float32)
    need = select_multi_workspace_size(B, Hq, Hkv, d, nq, s_max, k_max)
    if ws is None:
        ws = workspace(need, q.device)
    _check(lib().bd_select_multi(_DTYPE[q.dtype], B, Hq, Hkv, d, _ptr(q), _strides(q, 3), nq,
                                 _ptr(k), _strides(k, 3), k.shape[1], _ptr(s_len), s_max,
                                 _ptr(k_sel), k_max, float(sm_scale), _ptr(idx_out),
                                 _ptr(score_out), _ptr(ws), 0 if ws is None else ws.numel(),
                                 _stream()))
    return idx_out


def attn_workspace_size(dtype, B, Hq, Hkv, d, q, n_rows, p_max) -> int:
    return int(lib().bd_attn_workspace_size(_DTYPE.get(dtype, dtype), B, Hq, Hkv, d, q, n_rows, p_max))


def attn_packed(q, pk, pv, p_len, p_max: int, wk, wv, bl: int, sm_scale: float, out=None,
                lse=None, row_ids=None, ws=None, mask_mode: str = "block_causal"):
    """Packed block-diffusion attention; returns out [B, q, Hq, d].  Any
    ``mask_mode`` other than "block_causal" calls bd_attn_packed_masked."""
    q = _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, q, Hq, d]")
    B, nqry, Hq, d = q.shape
    pk = _dev(pk, "pk")
    Hkv = pk.shape[2] if pk.dim() == 4 else -1
    pk = _kv(pk, "pk", B, Hkv, d, q.dtype)
    pv = _kv(pv, "pv", B, Hkv, d, q.dtype)
    wk = _kv(wk, "wk", B, Hkv, d, q.dtype, min_len=nqry)
    wv = _kv(wv, "wv", B, Hkv, d, q.dtype, min_len=nqry)
    _pair(pk, pv, "pk", "pv")
    _pair(wk, wv, "wk", "wv")
    p_len = _rows(p_len, "p_len", B)
    rid = _i32(row_ids, "row_ids") if row_ids is not None else None
    n_rows = B if rid is None else rid.numel()
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    need = attn_workspace_size(q.dtype, B, Hq, Hkv, d, nqry, n_rows, p_max)
    if ws is None:
        ws = workspace(need, q.device)
    lse = _buf(lse, "lse", (B, Hq, nqry), torch.float32)
    tail = (_ptr(rid), n_rows, _ptr(q), _strides(q, 3), _ptr(pk), _ptr(pv), _strides(pk, 3),
            pk.shape[1], _ptr(p_len), p_max, _ptr(wk), _ptr(wv), _strides(wk, 3),
            float(sm_scale), _ptr(out), _strides(out, 3), _ptr(lse), _ptr(ws),
            0 if ws is None else ws.numel(), _stream())
    if mask_mode == "block_causal":
        _check(lib().bd_attn_packed(_DTYPE[q.dtype], B, Hq, Hkv, d, nqry, bl, *tail))
    else:
        _check(lib().bd_attn_packed_masked(_DTYPE[q.dtype], B, Hq, Hkv, d, nqry, bl,
                                           MASK_MODES[mask_mode], *tail))
    return out


def attn_packed_noalloc(q, pk, pv, p_len, p_max: int, wk, wv, bl: int, sm_scale: float,
                        out=None, lse=None, row_ids=None):
    """bd_attn_packed_noalloc: attn_packed with the scratch in the library's
    own device array (no workspace; allocates nothing when ``out`` is
    given).  Returns out [B, q, Hq, d]."""
    q = _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, q, Hq, d]")
    B, nqry, Hq, d = q.shape
    pk = _dev(pk, "pk")
    Hkv = pk.shape[2] if pk.dim() == 4 else -1
    pk = _kv(pk, "pk", B, Hkv, d, q.dtype)
    pv = _kv(pv, "pv", B, Hkv, d, q.dtype)
    wk = _kv(wk, "wk", B, Hkv, d, q.dtype, min_len=nqry)
    wv = _kv(wv, "wv", B, Hkv, d, q.dtype, min_len=nqry)
    _pair(pk, pv, "pk", "pv")
    _pair(wk, wv, "wk", "wv")
    p_len = _rows(p_len, "p_len", B)
    rid = _i32(row_ids, "row_ids") if row_ids is not None else None
    n_rows = B if rid is None else rid.numel()
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    lse = _buf(lse, "lse", (B, Hq, nqry), torch.float32)
    _check(lib().bd_attn_packed_noalloc(
        _DTYPE[q.dtype], B, Hq, Hkv, d, nqry, bl, _ptr(rid), n_rows, _ptr(q), _strides(q, 3),
        _ptr(pk), _ptr(pv), _strides(pk, 3), pk.shape[1], _ptr(p_len), p_max, _ptr(wk), _ptr(wv),
        _strides(wk, 3), float(sm_scale), _ptr(out), _strides(out, 3), _ptr(lse), _stream()))
    return out


def attn_block_table_workspace_size(dtype, Hq: int, Hkv: int, d: int, q: int, n_items: int,
                                    kv_max: int) -> int:
    return int(lib().bd_attn_block_table_workspace_size(_DTYPE.get(dtype, dtype), Hq, Hkv, d, q,
                                                        n_items, kv_max))


def attn_block_table(q, kv_k, kv_v, items, table, kv_max: int, wk, wv, bl: int,
                     sm_scale: float, out=None, lse=None, ws=None):
    """Block-table attention (bd_attn_block_table).  q [B, q, Hq, d]; kv_k /
    kv_v the paged store [n_pages, page, Hkv, d]; items int32 [n_items, 5]
    (row, q_begin, q_end, table_off, kv_len) in dispatch order; table int32
    [n_table] page ids; wk / wv [B, q, Hkv, d].  Outputs no item covers are
    left as they are in ``out``.  Returns out."""
    q = _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, q, Hq, d]")
    B, nqry, Hq, d = q.shape
    kv_k = _dev(kv_k, "kv_k")
    if kv_k.dim() != 4:
        raise ValueError("kv_k must be [n_pages, page, Hkv, d]")
    n_pages, page, Hkv = kv_k.shape[0], kv_k.shape[1], kv_k.shape[2]
    kv_k = _kv(kv_k, "kv_k", n_pages, Hkv, d, q.dtype)
    kv_v = _kv(kv_v, "kv_v", n_pages, Hkv, d, q.dtype)
    _pair(kv_k, kv_v, "kv_k", "kv_v")
    wk = _kv(wk, "wk", B, Hkv, d, q.dtype, min_len=nqry)
    wv = _kv(wv, "wv", B, Hkv, d, q.dtype, min_len=nqry)
    _pair(wk, wv, "wk", "wv")
    items = _i32(items, "items")
    if items.dim() != 2 or items.shape[1] != 5:
        raise ValueError("items must be int32 [n_items, 5]")
    table = _i32(table, "table")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    lse = _buf(lse, "lse", (B, Hq, nqry), torch.float32)
    n_items = items.shape[0]
    need = attn_block_table_workspace_size(q.dtype, Hq, Hkv, d, nqry, n_items, kv_max)
    if ws is None:
        ws = workspace(need, q.device)
    _check(lib().bd_attn_block_table(
        _DTYPE[q.dtype], B, Hq, Hkv, d, nqry, bl, _ptr(items), n_items, _ptr(table), table.numel(),
        _ptr(kv_k), _ptr(kv_v), _strides(kv_k, 3), n_pages, page, int(kv_max), _ptr(q),
        _strides(q, 3), _ptr(wk), _ptr(wv), _strides(wk, 3), float(sm_scale), _ptr(out),
        _strides(out, 3), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return out


def attn_dual_workspace_size(dtype, B: int, Hq: int, Hkv: int, d: int, q: int, n_a: int,
                             p_max_a: int, n_b: int, p_max_b: int) -> int:
    return int(lib().bd_attn_dual_workspace_size(_DTYPE.get(dtype, dtype), B, Hq, Hkv, d, q, n_a,
                                                 p_max_a, n_b, p_max_b))


def attn_packed_dual(q, src_a, src_b, wk, wv, bl: int, sm_scale: float, out=None, lse=None,
                     ws=None):
    """bd_attn_packed over two row lists in one launch.  src_a and src_b are
    (rows, pk, pv, p_len, p_max) tuples: the rows of each list attend over
    that list's prefix (e.g. the cache for dense rows, the pool for sparse
    rows).  Returns out [B, q, Hq, d]."""
    q = _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, q, Hq, d]")
    B, nqry, Hq, d = q.shape
    wk = _dev(wk, "wk")
    Hkv = wk.shape[2] if wk.dim() == 4 else -1
    wk = _kv(wk, "wk", B, Hkv, d, q.dtype, min_len=nqry)
    wv = _kv(wv, "wv", B, Hkv, d, q.dtype, min_len=nqry)
    _pair(wk, wv, "wk", "wv")
    srcs = []
    for tag, (rows, pk, pv, p_len, p_max) in (("a", src_a), ("b", src_b)):
        pk = _kv(pk, "pk_" + tag, B, Hkv, d, q.dtype)
        pv = _kv(pv, "pv_" + tag, B, Hkv, d, q.dtype)
        _pair(pk, pv, "pk_" + tag, "pv_" + tag)
        srcs.append((_i32(rows, "rows_" + tag), pk, pv, _rows(p_len, "p_len_" + tag, B), int(p_max)))
    (ra, pka, pva, pla, pma), (rb, pkb, pvb, plb, pmb) = srcs
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q's shape and dtype")
    need = attn_dual_workspace_size(q.dtype, B, Hq, Hkv, d, nqry, ra.numel(), pma, rb.numel(), pmb)
    if ws is None:
        ws = workspace(need, q.device)
    lse = _buf(lse, "lse", (B, Hq, nqry), torch.float32)
    _check(lib().bd_attn_packed_dual(
        _DTYPE[q.dtype], B, Hq, Hkv, d, nqry, bl, _ptr(q), _strides(q, 3),
        _ptr(ra), ra.numel(), _ptr(pka), _ptr(pva), _strides(pka, 3), pka.shape[1], _ptr(pla), pma,
        _ptr(rb), rb.numel(), _ptr(pkb), _ptr(pvb), _strides(pkb, 3), pkb.shape[1], _ptr(plb), pmb,
        _ptr(wk), _ptr(wv), _strides(wk, 3), float(sm_scale), _ptr(out), _strides(out, 3),
        _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return out


def qkv_rope_write(x, w, rope_pos, Hq: int, Hkv: int, q_out, k_cache, v_cache, dst_pos,
                   rope_base: float = 10000.0):
    """Fused QKV projection + RoPE + cache write.  x [B, q, Dm]; w
    [(Hq + 2 Hkv) * d, Dm]; q_out [B, q, Hq, d]; k_cache / v_cache
    [B, C, Hkv, d] (shared strides).  Returns q_out."""
    x, w = _dev(x, "x"), _dev(w, "w")
    q_out, k_cache, v_cache = _dev(q_out, "q_out"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache")
    if k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    for t, name in ((w, "w"), (q_out, "q_out"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != x.dtype:
            raise ValueError(f"{name} must be {x.dtype} like x, got {t.dtype}")
    if x.dim() != 3 or q_out.dim() != 4:
        raise ValueError("x must be [B, q, Dm] and q_out [B, q, Hq, d]")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    B, nq, Dm = x.shape
    d = q_out.shape[3]
    if tuple(w.shape) != ((Hq + 2 * Hkv) * d, Dm):
        raise ValueError(f"w must be [{(Hq + 2 * Hkv) * d}, {Dm}]")
    if tuple(q_out.shape) != (B, nq, Hq, d):
        raise ValueError(f"q_out must be [{B}, {nq}, {Hq}, {d}]")
    if k_cache.dim() != 4 or k_cache.shape[0] != B or tuple(k_cache.shape[2:]) != (Hkv, d) or \
            k_cache.shape != v_cache.shape:
        raise ValueError(f"k_cache / v_cache must be [{B}, C, {Hkv}, {d}]")
    rope_pos, dst_pos = _rows(rope_pos, "rope_pos", B), _rows(dst_pos, "dst_pos", B)
    _check(lib().bd_qkv_rope_write(_DTYPE[x.dtype], B, nq, Dm, Hq, Hkv, d, _ptr(x), _strides(x, 2),
                                   _ptr(w), _ptr(rope_pos), float(rope_base), _ptr(q_out),
                                   _strides(q_out, 3), _ptr(k_cache), _ptr(v_cache),
                                   _strides(k_cache, 3), k_cache.shape[1], _ptr(dst_pos), _stream()))
    return q_out


def mask_materialize(B: int, C: int, q: int, bl: int, o, mask_mode: str = "block_causal"):
    o = _rows(o, "o", B)
    out = torch.empty((B, q, C), dtype=torch.uint8, device=o.device)
    _check(lib().bd_mask_materialize(B, C, q, bl, MASK_MODES[mask_mode], _ptr(o), _ptr(out),
                                     _stream()))
    return out


# ---------------------------------------------------------------------------
# Device check mode: each function ORs BD_CHECK_* bits into ``status`` (a
# one-element int32 GPU tensor the caller clears) on the current stream.

def new_status(device=None) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device or "cuda")


def check_names(status: torch.Tensor) -> list[str]:
    """Names of the bits set in a status word (reads it on the host)."""
    v = int(status.item()) & 0xFFFFFFFF
    return [n for n, bit in CHECK_BITS.items() if v & bit]


def _status(st):
    if not isinstance(st, torch.Tensor) or not st.is_cuda or st.dtype != torch.int32 or st.numel() < 1:
        raise ValueError("status must be an int32 GPU tensor with at least one element")
    return st


def check_attn(status, B: int, p_len, p_max: int, p_cap: int, p_hi: int | None = None, row_ids=None):
    """Row ids in [0, B) and p_len in [0, min(p_max, p_cap, p_hi)]."""
    p_len = _rows(p_len, "p_len", B)
    rid = _i32(row_ids, "row_ids") if row_ids is not None else None
    n = B if rid is None else rid.numel()
    hi = p_cap if p_hi is None else p_hi
    _check(lib().bd_check_attn(B, _ptr(rid), n, _ptr(p_len), p_max, p_cap, hi, _ptr(_status(status)),
                               _stream()))


def check_scatter(status, B: int, q: int, t: int, data_cap: int, o, aliased: bool, row_ids=None):
    """o_b in [0, data_cap - q]; aliased: also o_b + q <= t or o_b == t."""
    o = _rows(o, "o", B)
    rid = _i32(row_ids, "row_ids") if row_ids is not None else None
    n = B if rid is None else rid.numel()
    _check(lib().bd_check_scatter(B, q, t, data_cap, _ptr(o), _ptr(rid), n, int(bool(aliased)),
                                  _ptr(_status(status)), _stream()))


def check_gather(status, idx, k_cnt, src_cap: int):
    """k_cnt in [0, k_max]; idx of the copied slots in [0, src_cap)."""
    idx = _i32(idx, "idx")
    if idx.dim() != 3:
        raise ValueError("idx must be [B, Hkv, k_max]")
    B, Hkv, k_max = idx.shape
    k_cnt = _rows(k_cnt, "k_cnt", B)
    _check(lib().bd_check_gather(B, Hkv, _ptr(idx), k_max, _ptr(k_cnt), src_cap,
                                 _ptr(_status(status)), _stream()))


def check_select(status, s_len, s_max: int, k_cap: int, k_sel, k_max: int):
    """s_len in [0, min(s_max, k_cap)] and k_sel in [0, k_max]."""
    B = s_len.numel()
    s_len, k_sel = _rows(s_len, "s_len", B), _rows(k_sel, "k_sel", B)
    _check(lib().bd_check_select(B, _ptr(s_len), s_max, k_cap, _ptr(k_sel), k_max,
                                 _ptr(_status(status)), _stream()))


def check_block_table(status, B: int, q: int, items, table, n_pages: int, page: int, kv_max: int):
    """Items' rows, query ranges, key counts, table ranges and page ids."""
    items = _i32(items, "items")
    if items.dim() != 2 or items.shape[1] != 5:
        raise ValueError("items must be int32 [n_items, 5]")
    table = _i32(table, "table")
    _check(lib().bd_check_block_table(B, q, _ptr(items), items.shape[0], _ptr(table), table.numel(),
                                      n_pages, page, kv_max, _ptr(_status(status)), _stream()))
