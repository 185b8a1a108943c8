"""Host-side tests of the C-ABI (no GPU needed).

The library loads, exports every function the header declares, and every
argument-validation path returns its documented status before any HIP
call (so none of these calls launches anything).
"""
import ctypes

import pytest

from sparse_kv_cache_bd_amd import bdattn as bd

I3 = ctypes.c_int64 * 3
I4 = ctypes.c_int64 * 4
FAKE = ctypes.c_void_p(0x100000)       # 16-byte aligned, never dereferenced
FAKE2 = ctypes.c_void_p(0x200000)
MISALIGNED = ctypes.c_void_p(0x100008)


@pytest.fixture(scope="module")
def L():
    return bd.lib()


def test_exports_every_header_function(L):
    names = bd.header_functions()
    assert len(names) == 25
    for n in names:
        assert hasattr(L, n), n


def test_version(L):
    assert bd.version().startswith("libbdattn")
    assert "gfx950" in bd.version()


def _scatter(L, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, Hkv=8, d=128, q=64, n_layers=1, pk=FAKE, pv=FAKE2,
             ps=I4(0, 4096 * 1024, 1024, 128), pcap=4096, t=4032, dk=FAKE, dv=FAKE2,
             ds=I4(0, 4096 * 1024, 1024, 128), dcap=4096, o=FAKE, rid=None, n_rows=2)
    a.update(kw)
    return L.bd_kv_scatter(a["dtype"], a["B"], a["Hkv"], a["d"], a["q"], a["n_layers"], a["pk"],
                           a["pv"], a["ps"], a["pcap"], a["t"], a["dk"], a["dv"], a["ds"],
                           a["dcap"], a["o"], a["rid"], a["n_rows"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), bd.BD_ERR_UNSUPPORTED),
    (dict(Hkv=0), bd.BD_ERR_INVALID_ARG),
    (dict(n_rows=1), bd.BD_ERR_INVALID_ARG),            # row_ids NULL needs n_rows == B
    (dict(d=4), bd.BD_ERR_UNSUPPORTED),                 # 8-byte rows
    (dict(o=None), bd.BD_ERR_INVALID_ARG),
    (dict(pk=None), bd.BD_ERR_INVALID_ARG),
    (dict(dv=None), bd.BD_ERR_INVALID_ARG),             # V pointers must pair up
    (dict(t=4040), bd.BD_ERR_INVALID_ARG),              # window past present_cap
    (dict(ps=I4(0, 4096 * 1024, 1023, 128)), bd.BD_ERR_INVALID_ARG),   # stride not 16 B
    (dict(pk=MISALIGNED), bd.BD_ERR_INVALID_ARG),
])
def test_scatter_validation(L, kw, code):
    assert _scatter(L, **kw) == code
    assert bd.last_error().startswith("bd_kv_scatter")


def test_scatter_empty_is_ok(L):
    assert _scatter(L, B=0, n_rows=0) == bd.BD_OK
    assert _scatter(L, q=0) == bd.BD_OK


def _gather(L, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, Hkv=8, d=128, ks=FAKE, vs=FAKE2, ss=I3(1 << 20, 1024, 128),
             scap=1000, idx=FAKE, kmax=64, kcnt=FAKE, kp=FAKE, vp=FAKE2, pls=I3(65536, 1024, 128),
             pcap=64)
    a.update(kw)
    return L.bd_gather(a["dtype"], a["B"], a["Hkv"], a["d"], a["ks"], a["vs"], a["ss"], a["scap"],
                       a["idx"], a["kmax"], a["kcnt"], a["kp"], a["vp"], a["pls"], a["pcap"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=-1), bd.BD_ERR_UNSUPPORTED),
    (dict(idx=None), bd.BD_ERR_INVALID_ARG),
    (dict(vp=None), bd.BD_ERR_INVALID_ARG),
    (dict(pcap=63), bd.BD_ERR_INVALID_ARG),
    (dict(ss=I3(1 << 20, 1025, 128)), bd.BD_ERR_INVALID_ARG),
    (dict(kp=MISALIGNED), bd.BD_ERR_INVALID_ARG),
    (dict(B=70000), bd.BD_ERR_INVALID_ARG),
])
def test_gather_validation(L, kw, code):
    assert _gather(L, **kw) == code


def _select(L, ws_bytes=None, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, Hq=32, Hkv=8, d=128, q=FAKE, qs=I3(32 * 4096, 4096, 128),
             nq=32, mode=bd.BD_REP_MEAN, row=0, k=FAKE2, ks=I3(1 << 22, 1024, 128), kcap=4000,
             s_len=FAKE, s_max=4000, k_sel=FAKE, k_max=200, scale=0.088, idx=FAKE, score=None,
             ws=FAKE)
    a.update(kw)
    need = bd.select_workspace_size(a["B"], a["Hq"], a["Hkv"], a["d"], a["s_max"], a["k_max"])
    wsb = need if ws_bytes is None else ws_bytes
    return L.bd_select(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"], a["qs"], a["nq"],
                       a["mode"], a["row"], a["k"], a["ks"], a["kcap"], a["s_len"], a["s_max"],
                       a["k_sel"], a["k_max"], a["scale"], a["idx"], a["score"], a["ws"], wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=bd.BD_F32), bd.BD_ERR_UNSUPPORTED),
    (dict(d=64), bd.BD_ERR_UNSUPPORTED),
    (dict(Hq=30), bd.BD_ERR_INVALID_ARG),
    (dict(Hq=128, Hkv=8), bd.BD_ERR_UNSUPPORTED),
    (dict(mode=5), bd.BD_ERR_INVALID_ARG),
    (dict(mode=bd.BD_REP_ROW, row=32), bd.BD_ERR_INVALID_ARG),
    (dict(nq=0), bd.BD_ERR_INVALID_ARG),
    (dict(scale=float("nan")), bd.BD_ERR_INVALID_ARG),
    (dict(scale=-1.0), bd.BD_ERR_INVALID_ARG),
    (dict(idx=None), bd.BD_ERR_INVALID_ARG),
    (dict(k=MISALIGNED), bd.BD_ERR_INVALID_ARG),
    (dict(ws=None), bd.BD_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100010)), bd.BD_ERR_WORKSPACE),   # not 256-byte aligned
])
def test_select_validation(L, kw, code):
    assert _select(L, **kw) == code


def test_select_workspace_too_small(L):
    need = bd.select_workspace_size(2, 32, 8, 128, 4000, 200)
    assert need > 0
    assert _select(L, ws_bytes=need - 1) == bd.BD_ERR_WORKSPACE
    assert "need" in bd.last_error()


def _select_attn(L, ws_bytes=None, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, Hq=32, Hkv=8, d=128, q=FAKE, qs=I3(32 * 4096, 4096, 128),
             nq=32, mode=bd.BD_REP_MEAN, row=0, k=FAKE2, ks=I3(1 << 22, 1024, 128), v=FAKE2,
             vs=I3(1 << 22, 1024, 128), kcap=4000, s_len=FAKE, s_max=4000, k_sel=FAKE, k_max=200,
             scale=0.088, idx=FAKE, score=None, o=FAKE, ws=FAKE)
    a.update(kw)
    need = bd.select_attn_workspace_size(a["B"], a["Hq"], a["Hkv"], a["d"], a["s_max"], a["k_max"])
    wsb = need if ws_bytes is None else ws_bytes
    return L.bd_select_attn(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"], a["qs"], a["nq"],
                            a["mode"], a["row"], a["k"], a["ks"], a["v"], a["vs"], a["kcap"],
                            a["s_len"], a["s_max"], a["k_sel"], a["k_max"], a["scale"], a["idx"],
                            a["score"], a["o"], a["ws"], wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=bd.BD_F32), bd.BD_ERR_UNSUPPORTED),
    (dict(d=64), bd.BD_ERR_UNSUPPORTED),
    (dict(Hq=30), bd.BD_ERR_INVALID_ARG),
    (dict(o=None), bd.BD_ERR_INVALID_ARG),
    (dict(v=None), bd.BD_ERR_INVALID_ARG),
    (dict(vs=None), bd.BD_ERR_INVALID_ARG),
    (dict(v=MISALIGNED), bd.BD_ERR_INVALID_ARG),
    (dict(vs=I3(1 << 22, 1001, 128)), bd.BD_ERR_INVALID_ARG),   # row stride not a 16-byte multiple
    (dict(idx=None), bd.BD_ERR_INVALID_ARG),
    (dict(ws=None), bd.BD_ERR_WORKSPACE),
])
def test_select_attn_validation(L, kw, code):
    assert _select_attn(L, **kw) == code


def test_select_attn_workspace(L):
    """The output pass's partials come on top of bd_select's workspace: one
    G x d fp32 block per (row, KV head, 1024 prefix positions)."""
    base = bd.select_workspace_size(2, 32, 8, 128, 4000, 200)
    need = bd.select_attn_workspace_size(2, 32, 8, 128, 4000, 200)
    assert need >= base + 2 * 8 * 4 * 4 * 128 * 4
    assert _select_attn(L, ws_bytes=need - 1) == bd.BD_ERR_WORKSPACE
    assert _select_attn(L, ws_bytes=base) == bd.BD_ERR_WORKSPACE
    assert _select_attn(L, B=0) == bd.BD_OK


def _select_multi(L, ws_bytes=None, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, Hq=32, Hkv=8, d=128, q=FAKE, qs=I3(32 * 4096, 4096, 128),
             nq=32, k=FAKE2, ks=I3(1 << 22, 1024, 128), kcap=4000, s_len=FAKE, s_max=4000,
             k_sel=FAKE, k_max=200, scale=0.088, idx=FAKE, score=None, ws=FAKE)
    a.update(kw)
    need = bd.select_multi_workspace_size(a["B"], a["Hq"], a["Hkv"], a["d"], a["nq"], a["s_max"],
                                          a["k_max"])
    wsb = need if ws_bytes is None else ws_bytes
    return L.bd_select_multi(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"], a["qs"],
                             a["nq"], a["k"], a["ks"], a["kcap"], a["s_len"], a["s_max"],
                             a["k_sel"], a["k_max"], a["scale"], a["idx"], a["score"], a["ws"],
                             wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=bd.BD_F32), bd.BD_ERR_UNSUPPORTED),
    (dict(d=64), bd.BD_ERR_UNSUPPORTED),
    (dict(Hq=30), bd.BD_ERR_INVALID_ARG),
    (dict(nq=33), bd.BD_ERR_UNSUPPORTED),               # 33 * 4 columns > 128
    (dict(Hq=64, Hkv=8, nq=17), bd.BD_ERR_UNSUPPORTED),  # 17 * 8 > 128
    (dict(nq=0), bd.BD_ERR_INVALID_ARG),
    (dict(scale=float("nan")), bd.BD_ERR_INVALID_ARG),
    (dict(idx=None), bd.BD_ERR_INVALID_ARG),
    (dict(q=MISALIGNED), bd.BD_ERR_INVALID_ARG),
    (dict(qs=I3(32 * 4096, 4096, 100)), bd.BD_ERR_INVALID_ARG),   # head stride not 16 B
    (dict(ws=None), bd.BD_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100010)), bd.BD_ERR_WORKSPACE),
])
def test_select_multi_validation(L, kw, code):
    assert _select_multi(L, **kw) == code


def test_select_multi_workspace(L):
    need = bd.select_multi_workspace_size(2, 32, 8, 128, 32, 4000, 200)
    assert need > 0
    assert _select_multi(L, ws_bytes=need - 1) == bd.BD_ERR_WORKSPACE
    assert _select_multi(L, B=0) == bd.BD_OK and _select_multi(L, k_max=0) == bd.BD_OK
    # more prefix needs more chunk partials and scores; longer than 32K adds the ranking histograms
    assert bd.select_multi_workspace_size(1, 32, 8, 128, 32, 40000, 200) > \
        bd.select_multi_workspace_size(1, 32, 8, 128, 32, 32768, 200) > need // 2 > 0


def test_workspace_sizes_monotone():
    a = bd.select_workspace_size(4, 32, 8, 128, 32768, 1638)
    b = bd.select_workspace_size(4, 32, 8, 128, 65536, 1638)
    assert 0 < a < b
    # few units: the attention splits its prefix and needs a workspace
    assert bd.attn_workspace_size(bd.BD_BF16, 1, 32, 8, 128, 32, 1, 6554) > 0
    # many units: one chunk per unit; the workspace only holds the longest-first
    # row order (64 int32 rounded up to 256 bytes), no partial results
    assert bd.attn_workspace_size(bd.BD_BF16, 64, 32, 8, 128, 128, 64, 16384) == 256
    # units that fit the GPU at once: neither an order nor partial results
    assert bd.attn_workspace_size(bd.BD_BF16, 16, 32, 8, 128, 128, 16, 900) == 0


def _attn(L, ws_bytes=None, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, Hq=32, Hkv=8, d=128, q=64, bl=32, rid=None, n_rows=2,
             Q=FAKE, qs=I3(64 * 4096, 4096, 128), pk=FAKE, pv=FAKE2, ps=I3(1 << 22, 1024, 128),
             pcap=4096, plen=FAKE, pmax=4000, wk=FAKE, wv=FAKE2, wsd=I3(1 << 22, 1024, 128),
             scale=0.088, out=FAKE2, os=I3(64 * 4096, 4096, 128), lse=None, ws=FAKE)
    a.update(kw)
    need = bd.attn_workspace_size(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"],
                                  a["n_rows"], a["pmax"])
    wsb = need if ws_bytes is None else ws_bytes
    return L.bd_attn_packed(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"], a["bl"],
                            a["rid"], a["n_rows"], a["Q"], a["qs"], a["pk"], a["pv"], a["ps"],
                            a["pcap"], a["plen"], a["pmax"], a["wk"], a["wv"], a["wsd"],
                            a["scale"], a["out"], a["os"], a["lse"], a["ws"], wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), bd.BD_ERR_UNSUPPORTED),
    (dict(d=96), bd.BD_ERR_UNSUPPORTED),
    (dict(Hq=33), bd.BD_ERR_INVALID_ARG),
    (dict(bl=0), bd.BD_ERR_INVALID_ARG),
    (dict(n_rows=1), bd.BD_ERR_INVALID_ARG),
    (dict(plen=None), bd.BD_ERR_INVALID_ARG),
    (dict(pk=None), bd.BD_ERR_INVALID_ARG),
    (dict(wv=MISALIGNED), bd.BD_ERR_INVALID_ARG),
    (dict(os=I3(64 * 4096, 4096, 129)), bd.BD_ERR_INVALID_ARG),
    (dict(scale=0.0), bd.BD_ERR_INVALID_ARG),
    (dict(ws=None), bd.BD_ERR_WORKSPACE),
])
def test_attn_validation(L, kw, code):
    assert _attn(L, **kw) == code


def _attn_noalloc(L, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, Hq=32, Hkv=8, d=128, q=64, bl=32, rid=None, n_rows=2,
             Q=FAKE, qs=I3(64 * 4096, 4096, 128), pk=FAKE, pv=FAKE2, ps=I3(1 << 22, 1024, 128),
             pcap=4096, plen=FAKE, pmax=4000, wk=FAKE, wv=FAKE2, wsd=I3(1 << 22, 1024, 128),
             scale=0.088, out=FAKE2, os=I3(64 * 4096, 4096, 128), lse=None)
    a.update(kw)
    return L.bd_attn_packed_noalloc(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"], a["bl"],
                                    a["rid"], a["n_rows"], a["Q"], a["qs"], a["pk"], a["pv"],
                                    a["ps"], a["pcap"], a["plen"], a["pmax"], a["wk"], a["wv"],
                                    a["wsd"], a["scale"], a["out"], a["os"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), bd.BD_ERR_UNSUPPORTED),
    (dict(Hq=33), bd.BD_ERR_INVALID_ARG),
    (dict(n_rows=1), bd.BD_ERR_INVALID_ARG),
    (dict(plen=None), bd.BD_ERR_INVALID_ARG),
    (dict(wv=MISALIGNED), bd.BD_ERR_INVALID_ARG),
    (dict(scale=0.0), bd.BD_ERR_INVALID_ARG),
    (dict(B=0, n_rows=0), bd.BD_OK),
    (dict(q=0), bd.BD_OK),
])
def test_attn_noalloc_validation(L, kw, code):
    """The allocation-free variant validates exactly like bd_attn_packed."""
    assert _attn_noalloc(L, **kw) == code
    if code != bd.BD_OK:
        assert bd.last_error().startswith("bd_attn_packed_noalloc")


def test_attn_noalloc_rejects_oversized_scratch(L):
    """A call whose scratch exceeds the library's array is refused with
    BD_ERR_WORKSPACE before any HIP call (the size comes from the plan)."""
    cap = bd.noalloc_scratch_bytes()
    assert cap == 32 << 20
    # 255 units (one short of a block per CU) over 1024-key prefixes: each is
    # cut in two chunks, whose partials (255 x 2 x 256 columns) pass 32 MB;
    # split plans are largest just below one unit per CU
    kw = dict(B=255, n_rows=255, Hq=8, Hkv=1, q=32, pmax=1024, pcap=1024)
    need = bd.attn_workspace_size(bd.BD_BF16, 255, 8, 1, 128, 32, 255, 1024)
    assert need > cap
    assert _attn_noalloc(L, **kw) == bd.BD_ERR_WORKSPACE
    assert "scratch" in bd.last_error() and str(need) in bd.last_error()


def _attn_bt(L, ws_bytes=None, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, Hq=32, Hkv=8, d=128, q=64, bl=32, items=FAKE, n_items=2,
             table=FAKE2, n_table=100, kv=FAKE, kvv=FAKE2, kvs=I3(128 * 1024, 1024, 128),
             n_pages=50, page=128, kv_max=4000, Q=FAKE, qs=I3(64 * 4096, 4096, 128), wk=FAKE,
             wv=FAKE2, wsd=I3(1 << 22, 1024, 128), scale=0.088, out=FAKE2,
             os=I3(64 * 4096, 4096, 128), lse=None, ws=FAKE)
    a.update(kw)
    need = bd.attn_block_table_workspace_size(a["dtype"], a["Hq"], a["Hkv"], a["d"], a["q"],
                                              a["n_items"], a["kv_max"])
    wsb = need if ws_bytes is None else ws_bytes
    return L.bd_attn_block_table(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"], a["bl"],
                                 a["items"], a["n_items"], a["table"], a["n_table"], a["kv"],
                                 a["kvv"], a["kvs"], a["n_pages"], a["page"], a["kv_max"], a["Q"],
                                 a["qs"], a["wk"], a["wv"], a["wsd"], a["scale"], a["out"], a["os"],
                                 a["lse"], a["ws"], wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=bd.BD_F32), bd.BD_ERR_UNSUPPORTED),       # MFMA path only
    (dict(d=64), bd.BD_ERR_UNSUPPORTED),
    (dict(Hq=24), bd.BD_ERR_UNSUPPORTED),                 # G = 3
    (dict(Hq=33), bd.BD_ERR_INVALID_ARG),
    (dict(page=96), bd.BD_ERR_INVALID_ARG),               # not a multiple of 64
    (dict(page=0), bd.BD_ERR_INVALID_ARG),
    (dict(n_items=-1), bd.BD_ERR_INVALID_ARG),
    (dict(items=None), bd.BD_ERR_INVALID_ARG),
    (dict(table=None), bd.BD_ERR_INVALID_ARG),
    (dict(kv=MISALIGNED), bd.BD_ERR_INVALID_ARG),
    (dict(kvs=I3(128 * 1024, 1024, 100)), bd.BD_ERR_INVALID_ARG),
    (dict(scale=float("inf")), bd.BD_ERR_INVALID_ARG),
    (dict(ws=None), bd.BD_ERR_WORKSPACE),
    (dict(n_items=0, items=None), bd.BD_OK),
    (dict(B=0), bd.BD_OK),
])
def test_attn_block_table_validation(L, kw, code):
    assert _attn_bt(L, **kw) == code
    if code != bd.BD_OK:
        assert bd.last_error().startswith("bd_attn_block_table")


def test_attn_block_table_workspace(L):
    # few items over long key lists: split partials, no row order (the
    # caller's order is kept)
    few = bd.attn_block_table_workspace_size(bd.BD_BF16, 32, 8, 128, 32, 4, 1638)
    assert few == bd.attn_workspace_size(bd.BD_BF16, 4, 32, 8, 128, 32, 4, 1638) > 0
    assert bd.attn_block_table_workspace_size(bd.BD_BF16, 32, 8, 128, 128, 64, 16384) == 0
    need = bd.attn_block_table_workspace_size(bd.BD_BF16, 32, 8, 128, 64, 2, 4000)
    assert need > 0
    assert _attn_bt(L, ws_bytes=need - 1) == bd.BD_ERR_WORKSPACE


def _attn_masked(L, mode, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, Hq=32, Hkv=8, d=128, q=64, bl=32, rid=None, n_rows=2,
             Q=FAKE, qs=I3(64 * 4096, 4096, 128), pk=FAKE, pv=FAKE2, ps=I3(1 << 22, 1024, 128),
             pcap=4096, plen=FAKE, pmax=4000, wk=FAKE, wv=FAKE2, wsd=I3(1 << 22, 1024, 128),
             scale=0.088, out=FAKE2, os=I3(64 * 4096, 4096, 128), lse=None, ws=FAKE)
    a.update(kw)
    need = bd.attn_workspace_size(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"],
                                  a["n_rows"], a["pmax"])
    return L.bd_attn_packed_masked(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"], a["bl"],
                                   mode, a["rid"], a["n_rows"], a["Q"], a["qs"], a["pk"], a["pv"],
                                   a["ps"], a["pcap"], a["plen"], a["pmax"], a["wk"], a["wv"],
                                   a["wsd"], a["scale"], a["out"], a["os"], a["lse"], a["ws"], need,
                                   None)


def test_attn_masked_validation(L):
    for mode in (-1, 3, 99):
        assert _attn_masked(L, mode) == bd.BD_ERR_INVALID_ARG
        assert "mask mode" in bd.last_error()
    # the other checks are those of bd_attn_packed
    assert _attn_masked(L, bd.BD_MASK_ISOLATED, Hq=30) == bd.BD_ERR_INVALID_ARG
    assert _attn_masked(L, bd.BD_MASK_SHARED_FIRST, Q=MISALIGNED) == bd.BD_ERR_INVALID_ARG
    assert _attn_masked(L, bd.BD_MASK_ISOLATED, B=0, n_rows=0) == bd.BD_OK


def test_attn_empty_is_ok(L):
    assert _attn(L, B=0, n_rows=0) == bd.BD_OK
    assert _attn(L, q=0) == bd.BD_OK


def _attn_dual(L, ws_bytes=None, **kw):
    a = dict(dtype=bd.BD_BF16, B=4, Hq=32, Hkv=8, d=128, q=64, bl=32,
             Q=FAKE, qs=I3(64 * 4096, 4096, 128),
             ra=FAKE, na=2, pka=FAKE, pva=FAKE2, psa=I3(1 << 22, 1024, 128), pcapa=4096,
             plena=FAKE, pmaxa=4000,
             rb=FAKE2, nb=2, pkb=FAKE2, pvb=FAKE, psb=I3(1 << 20, 1024, 128), pcapb=1024,
             plenb=FAKE2, pmaxb=200,
             wk=FAKE, wv=FAKE2, wsd=I3(1 << 22, 1024, 128), scale=0.088, out=FAKE2,
             os=I3(64 * 4096, 4096, 128), lse=None, ws=FAKE)
    a.update(kw)
    need = bd.attn_dual_workspace_size(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"],
                                       a["na"], a["pmaxa"], a["nb"], a["pmaxb"])
    wsb = need if ws_bytes is None else ws_bytes
    return L.bd_attn_packed_dual(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["q"], a["bl"],
                                 a["Q"], a["qs"], a["ra"], a["na"], a["pka"], a["pva"], a["psa"],
                                 a["pcapa"], a["plena"], a["pmaxa"], a["rb"], a["nb"], a["pkb"],
                                 a["pvb"], a["psb"], a["pcapb"], a["plenb"], a["pmaxb"], a["wk"],
                                 a["wv"], a["wsd"], a["scale"], a["out"], a["os"], a["lse"],
                                 a["ws"], wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), bd.BD_ERR_UNSUPPORTED),
    (dict(Hq=33), bd.BD_ERR_INVALID_ARG),
    (dict(nb=-1), bd.BD_ERR_INVALID_ARG),
    (dict(rb=None), bd.BD_ERR_INVALID_ARG),
    (dict(ra=None), bd.BD_ERR_INVALID_ARG),
    (dict(plenb=None), bd.BD_ERR_INVALID_ARG),
    (dict(pkb=None), bd.BD_ERR_INVALID_ARG),
    (dict(pvb=MISALIGNED), bd.BD_ERR_INVALID_ARG),
    (dict(psb=I3(1 << 20, 1024, 129)), bd.BD_ERR_INVALID_ARG),
    (dict(scale=0.0), bd.BD_ERR_INVALID_ARG),
    (dict(ws=None), bd.BD_ERR_WORKSPACE),
])
def test_attn_dual_validation(L, kw, code):
    assert _attn_dual(L, **kw) == code


def test_attn_dual_empty_and_one_list(L):
    assert _attn_dual(L, na=0, nb=0) == bd.BD_OK
    assert _attn_dual(L, q=0) == bd.BD_OK
    # an empty list needs neither rows nor a prefix source
    assert _attn_dual(L, na=0, ra=None, pka=None, pva=None, plena=None, nb=0, rb=None) == bd.BD_OK
    # the workspace is the one-list workspace of all rows and the longer prefix
    assert (bd.attn_dual_workspace_size(bd.BD_BF16, 64, 32, 8, 128, 128, 48, 8000, 16, 800)
            == bd.attn_workspace_size(bd.BD_BF16, 64, 32, 8, 128, 128, 64, 8000))


def test_mask_validation(L):
    assert L.bd_mask_materialize(2, 100, 200, 32, 0, FAKE, FAKE2, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_mask_materialize(2, 100, 64, 0, 0, FAKE, FAKE2, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_mask_materialize(2, 100, 64, 32, 0, None, FAKE2, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_mask_materialize(2, 100, 64, 32, 3, FAKE, FAKE2, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_mask_materialize(0, 100, 64, 32, 0, None, None, None) == bd.BD_OK


def _produce(L, **kw):
    a = dict(dtype=bd.BD_BF16, B=2, q=64, Dm=256, Hq=8, Hkv=2, d=128, x=FAKE,
             xs=(ctypes.c_int64 * 2)(64 * 256, 256), w=FAKE2, rope_pos=FAKE, base=10000.0,
             qo=FAKE, qs=I3(64 * 1024, 1024, 128), kc=FAKE, vc=FAKE2, cs=I3(1 << 20, 256, 128),
             cap=4096, dst=FAKE)
    a.update(kw)
    return L.bd_qkv_rope_write(a["dtype"], a["B"], a["q"], a["Dm"], a["Hq"], a["Hkv"], a["d"],
                               a["x"], a["xs"], a["w"], a["rope_pos"], a["base"], a["qo"],
                               a["qs"], a["kc"], a["vc"], a["cs"], a["cap"], a["dst"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=bd.BD_F32), bd.BD_ERR_UNSUPPORTED),
    (dict(d=64), bd.BD_ERR_UNSUPPORTED),
    (dict(Dm=96), bd.BD_ERR_UNSUPPORTED),                  # not a multiple of 64
    (dict(Dm=0), bd.BD_ERR_INVALID_ARG),
    (dict(base=1.0), bd.BD_ERR_INVALID_ARG),
    (dict(base=float("nan")), bd.BD_ERR_INVALID_ARG),
    (dict(w=None), bd.BD_ERR_INVALID_ARG),
    (dict(dst=None), bd.BD_ERR_INVALID_ARG),
    (dict(x=MISALIGNED), bd.BD_ERR_INVALID_ARG),
    (dict(cs=I3(1 << 20, 250, 128)), bd.BD_ERR_INVALID_ARG),   # row stride not 16 B
    (dict(B=0), bd.BD_OK),
    (dict(q=0, x=None), bd.BD_OK),
    (dict(Hq=4096, Hkv=2048, Dm=1024), bd.BD_ERR_UNSUPPORTED),              # W spans 2 GiB
    (dict(xs=(ctypes.c_int64 * 2)(1 << 30, 256)), bd.BD_ERR_UNSUPPORTED),  # x spans over 2 GiB
])
def test_producer_validation(L, kw, code):
    assert _produce(L, **kw) == code


def test_plain_c_client(tmp_path):
    """The public header is plain C: a C99 program includes it, links the
    library and gets the documented status codes from host-side validation
    (no kernel launches)."""
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    inc = os.path.dirname(bd.HEADER_PATH)
    libdir = os.path.dirname(bd.LIB_PATH)
    src = tmp_path / "client.c"
    src.write_text(r"""
#include <stdio.h>
#include <string.h>
#include "bdattn.h"
int main(void) {
  int64_t s3[3] = {0, 0, 0};
  if (strncmp(bd_version(), "libbdattn", 9) != 0) return 10;
  /* unknown dtype: unsupported, before any device work */
  if (bd_select(7, 1, 8, 2, 128, 0, s3, 1, BD_REP_MEAN, 0, 0, s3, 0, 0, 0, 0, 1, 0.1f, 0, 0, 0, 0,
                0) != BD_ERR_UNSUPPORTED) return 11;
  if (strlen(bd_last_error()) == 0) return 12;
  /* unknown mask mode */
  if (bd_attn_packed_masked(BD_BF16, 1, 8, 2, 128, 32, 32, 9, 0, 1, 0, s3, 0, 0, s3, 0, 0, 0, 0, 0,
                            s3, 0.1f, 0, s3, 0, 0, 0, 0) != BD_ERR_INVALID_ARG) return 13;
  /* empty calls succeed */
  if (bd_gather(BD_BF16, 0, 8, 128, 0, 0, s3, 0, 0, 0, 0, 0, 0, s3, 0, 0) != BD_OK) return 14;
  if (bd_qkv_rope_write(BD_BF16, 0, 32, 128, 4, 2, 128, 0, 0, 0, 0, 10000.f, 0, 0, 0, 0, 0, 0, 0,
                        0) != BD_OK) return 15;
  printf("ok\n");
  return 0;
}
""")
    exe = tmp_path / "client"
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", inc, str(src), "-L", libdir,
                        "-lbdattn", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


def test_check_validation(L):
    """The check functions validate their host arguments before any launch;
    empty calls do nothing."""
    S = FAKE2
    assert L.bd_check_attn(2, None, 2, FAKE, 10, 10, 10, None, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_attn(2, None, 3, FAKE, 10, 10, 10, S, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_attn(-1, None, 0, FAKE, 10, 10, 10, S, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_attn(2, None, 0, None, 10, 10, 10, None, None) == bd.BD_OK
    assert L.bd_check_scatter(2, 32, 96, 128, None, None, 2, 1, S, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_scatter(2, -1, 96, 128, FAKE, None, 2, 1, S, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_scatter(2, 32, 96, 128, FAKE, None, 0, 1, None, None) == bd.BD_OK
    assert L.bd_check_gather(2, 0, FAKE, 4, FAKE, 10, S, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_gather(70000, 1, FAKE, 4, FAKE, 10, S, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_gather(2, 8, FAKE, 4, None, 10, S, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_gather(2, 8, None, 0, None, 10, None, None) == bd.BD_OK
    assert L.bd_check_select(2, FAKE, 10, 10, FAKE, 5, None, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_select(0, None, 10, 10, None, 5, None, None) == bd.BD_OK
    assert L.bd_check_block_table(2, 64, FAKE, 2, FAKE, 10, 5, 96, 100, S, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_block_table(2, 64, None, 2, FAKE, 10, 5, 64, 100, S, None) == bd.BD_ERR_INVALID_ARG
    assert L.bd_check_block_table(2, 64, FAKE, 0, None, 0, 5, 64, 100, None, None) == bd.BD_OK
    assert bd.last_error() == ""
