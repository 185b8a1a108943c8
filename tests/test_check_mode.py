"""Device check mode: each out-of-contract per-row value sets its status
bit, and in-contract values leave the status word clear: those of the
serving-mix step (selection, gather, both attention row kinds, the aliased
scatter) and a valid block table.  The checks only read the values;
no operation is run on out-of-contract inputs here."""
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


def i32(*v):
    return torch.tensor(v, dtype=torch.int32, device="cuda")


def flags(bd, fn):
    st = bd.new_status()
    fn(st)
    torch.cuda.synchronize()
    return bd.check_names(st)


def test_attention_values(bd):
    note("check mode: attention")
    f = lambda p_len, **kw: flags(bd, lambda st: bd.check_attn(st, 4, p_len, 100, 150, **kw))
    assert f(i32(0, 10, 99, 100)) == []
    assert f(i32(0, -1, 99, 100)) == ["length"]
    assert f(i32(0, 10, 101, 100)) == ["length"]                 # past p_max
    assert f(i32(0, 10, 91, 90), p_hi=90) == ["length"]          # past the caller's bound (t)
    assert f(i32(0, 10, 90, 90), p_hi=90) == []
    assert f(i32(0, 10, 99, 100), row_ids=i32(3, 0, 4)) == ["row"]
    assert f(i32(0, -5, 99, 100), row_ids=i32(3, 0, -1)) == ["row"]   # row 1 not listed
    assert f(i32(0, -5, 99, 100), row_ids=i32(1, 7)) == ["row", "length"]


def test_scatter_values(bd):
    note("check mode: scatter")
    f = lambda o, aliased, **kw: flags(bd, lambda st: bd.check_scatter(st, 4, 32, 96, 128, o, aliased, **kw))
    assert f(i32(0, 64, 96, 10), True) == []                 # o + q <= t, or o == t
    assert f(i32(0, 64, 96, 10), False) == []
    assert f(i32(0, 80, 96, 10), True) == ["alias"]          # target [80, 112) overlaps the tail [96, 128)
    assert f(i32(0, 80, 96, 10), False) == []                 # separate tensors: allowed
    assert f(i32(-3, 64, 96, 10), True) == ["offset"]
    assert f(i32(0, 97, 96, 10), False) == ["offset"]         # 97 + 32 > 128
    assert f(i32(0, 0, 0, 0), True, row_ids=i32(2, 4)) == ["row"]


def test_gather_values(bd):
    note("check mode: gather")
    idx = torch.full((2, 3, 8), -1, dtype=torch.int32, device="cuda")
    idx[:, :, :5] = torch.arange(5, dtype=torch.int32, device="cuda") * 7
    f = lambda cnt: flags(bd, lambda st: bd.check_gather(st, idx, cnt, 40))
    assert f(i32(5, 3)) == []                 # -1 padding past k_cnt is fine
    assert f(i32(5, 0)) == []
    assert f(i32(6, 3)) == ["index"]          # slot 5 holds -1
    assert f(i32(9, 3)) == ["length", "index"]
    assert f(i32(-1, 3)) == ["length"]
    idx[1, 2, 4] = 40                          # == src_cap
    assert f(i32(5, 5)) == ["index"]
    assert f(i32(5, 4)) == []


def test_select_values(bd):
    note("check mode: select")
    f = lambda s, k: flags(bd, lambda st: bd.check_select(st, s, 1000, 900, k, 50))
    assert f(i32(900, 0, 10), i32(50, 0, 3)) == []
    assert f(i32(901, 0, 10), i32(50, 0, 3)) == ["length"]     # past k_cap
    assert f(i32(900, 0, 10), i32(51, 0, 3)) == ["length"]
    assert f(i32(900, -2, 10), i32(50, 0, 3)) == ["length"]


def test_block_table_values(bd):
    note("check mode: block table")
    table = i32(3, 0, 1, 2, 4)
    good = [(0, 0, 64, 0, 200), (1, 32, 64, 4, 64)]

    def f(items, n_pages=5):
        return flags(bd, lambda st: bd.check_block_table(st, 2, 64, i32(*sum(items, ())).view(-1, 5),
                                                         table, n_pages, 64, 300))
    assert f(good) == []
    assert f([(2, 0, 64, 0, 200)]) == ["row"]
    assert f([(0, 64, 80, 0, 200)]) == ["queries"]
    assert f([(0, 10, 10, 0, 200)]) == ["queries"]
    assert f([(0, 0, 64, 0, 301)]) == ["length"]               # clamped to 300: its 5 pages fit the table
    assert f([(0, 0, 64, 2, 200)]) == ["page"]                 # 4 pages from entry 2 run past the table
    assert f([(0, 0, 64, -1, 0)]) == ["page"]
    assert f(good, n_pages=4) == ["page"]                       # page id 4
    assert f([(0, 0, 64, 0, 0), (1, 0, 1, 5, 0)]) == []         # empty key lists need no pages


def test_real_workloads_are_clean(bd):
    """The serving-mix step's values pass every check, before and after the
    step (the selection's indices feed the gather check)."""
    from sparse_kv_cache_bd_amd.pipeline import BlockDiffusionStep
    note("check mode: serving mix is clean")
    wl = synth.serving_mix(seed=5, B=24, p_lo=1024, p_hi=16384)
    Kc, Vc, Q, o = wl.Kc.cuda(), wl.Vc.cuda(), wl.Q.cuda(), wl.o.cuda()
    step = BlockDiffusionStep(Kc, Vc, Q, o, wl.bl, wl.sm_scale, sparse_rows=wl.sparse_rows,
                              dense_rows=wl.dense_rows, s_len=wl.s_len, k_sel=wl.k_sel,
                              p_max_dense=int(wl.o.max()), k_max=wl.k_max, s_max=wl.s_max)
    st = bd.new_status()
    bd.check_select(st, step.s_len, wl.s_max, wl.C, step.k_sel, wl.k_max)
    bd.check_attn(st, wl.B, o, step.p_max_dense, wl.C, p_hi=wl.t, row_ids=step.dense_rows)
    bd.check_scatter(st, wl.B, wl.q, wl.t, wl.C, o, aliased=True)
    step.run()
    bd.check_gather(st, step.idx, step.k_eff, wl.C)
    bd.check_attn(st, wl.B, step.k_eff, wl.k_max, wl.k_max, row_ids=step.sparse_rows)
    torch.cuda.synchronize()
    assert bd.check_names(st) == []
