"""GPU parity of bd_attn_block_table (Flash-dLLM, Scheduled Flash Attention,
Fig. 3(b)): work items over a paged KV store, in the caller's order, against
the float64 oracle's block_table_attention.

The store's pages sit at shuffled physical slots; slots no table entry
names, and the positions past a row's keys on its last page, hold NaN, so
a read of anything outside an item's key list shows in the output.
Outputs no item covers hold a sentinel that must survive the call.
"""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import bits, check_attention, note
from oracle import bd_oracle as orc

pytestmark = pytest.mark.gpu

SENTINEL = -7.0


@pytest.fixture(scope="module")
def bd():
    from sparse_kv_cache_bd_amd import bdattn
    bdattn.lib()
    return bdattn


def paged(wl, page, seed, spare=5):
    """The rows' prefixes [0, o_b) cut into pages of `page` keys, placed at
    shuffled slots of a NaN-filled store with `spare` unused slots.
    Returns (KP, VP, table, items) as CPU tensors; items one per row, all
    queries, in row order."""
    P = [int(v) for v in wl.o]
    n_pages = [math.ceil(p / page) for p in P]
    total = sum(n_pages) + spare
    slots = np.random.default_rng(seed).permutation(total)
    KP = torch.full((total, page, wl.Hkv, wl.d), float("nan"), dtype=wl.Kc.dtype)
    VP = torch.full_like(KP, float("nan"))
    table, items, e = [], [], 0
    for b, p in enumerate(P):
        off = len(table)
        for j in range(n_pages[b]):
            n = min(page, p - j * page)
            s = int(slots[e])
            KP[s, :n] = wl.Kc[b, j * page:j * page + n]
            VP[s, :n] = wl.Vc[b, j * page:j * page + n]
            table.append(s)
            e += 1
        items.append((b, 0, wl.q, off, p))
    return KP, VP, torch.tensor(table, dtype=torch.int32), torch.tensor(items, dtype=torch.int32)


def run_gpu(bd, wl, KP, VP, items, table, kv_max, out=None, lse=None):
    t = wl.t
    Kc, Vc = wl.Kc.cuda(), wl.Vc.cuda()
    if out is None:
        out = torch.full((wl.B, wl.q, wl.Hq, wl.d), SENTINEL, dtype=wl.Q.dtype, device="cuda")
    bd.attn_block_table(wl.Q.cuda(), KP.cuda(), VP.cuda(), items.cuda(), table.cuda(), kv_max,
                        Kc[:, t:], Vc[:, t:], wl.bl, wl.sm_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out


def oracle(wl, KP, VP, items, table, kv_max=None):
    t = wl.t
    return orc.block_table_attention(wl.Q, KP, VP, items.numpy(), table.numpy(), KP.shape[1],
                                     wl.Kc[:, t:], wl.Vc[:, t:], wl.bl, wl.sm_scale, kv_max=kv_max)


def check_items(out, ref, items, q, label):
    """Covered (row, query) outputs against the oracle; every other output
    still holds the sentinel."""
    covered = np.zeros((out.shape[0], q), bool)
    for b, q0, q1, _, _ in items.tolist():
        covered[b, q0:min(q1, q)] = True
    g = out.detach().cpu().double().numpy()
    for b in range(out.shape[0]):
        if covered[b].any():
            qs = np.nonzero(covered[b])[0]
            check_attention(out[b:b + 1, torch.from_numpy(qs).cuda()], ref[b:b + 1, qs], torch.bfloat16,
                            label=f"{label} row {b}")
        assert (g[b][~covered[b]] == SENTINEL).all(), f"{label}: row {b}: uncovered output written"


@pytest.mark.parametrize("page", [64, 128, 256])
def test_shuffled_pages(bd, page):
    """Ragged prefixes (not multiples of the page) on shuffled pages; items
    in a random order with one row left out."""
    note(f"block table: shuffled pages, page={page}")
    wl = synth.serving_mix(seed=11, B=6, p_lo=500, p_hi=3000, W=4, sparse_above=10 ** 9)
    KP, VP, table, items = paged(wl, page, seed=page)
    # key counts below the rows' prefixes, not multiples of 32: keys past
    # kv_len on the last page hold real values and must stay invisible
    items[:, 4] -= torch.tensor([(7 * b) % 29 + 1 for b in range(wl.B)], dtype=torch.int32)
    order = torch.from_numpy(np.random.default_rng(page).permutation(wl.B))
    items = items[order][:-1].contiguous()          # the last row in this order is left out
    kv_max = int(wl.o.max())
    out = run_gpu(bd, wl, KP, VP, items, table, kv_max)
    ref, _ = oracle(wl, KP, VP, items, table)
    check_items(out, ref, items, wl.q, f"page {page}")


def test_contiguous_table_equals_packed(bd):
    """Pages of a row in order at consecutive slots: bd_attn_packed's
    arithmetic on the same keys, so the outputs and LSE agree bit for bit."""
    note("block table: contiguous table vs bd_attn_packed")
    wl = synth.serving_mix(seed=12, B=10, p_lo=300, p_hi=4000, W=4, sparse_above=10 ** 9)
    page = 64
    P = [int(v) for v in wl.o]
    n_pages = [math.ceil(p / page) for p in P]
    KP = torch.zeros((sum(n_pages), page, wl.Hkv, wl.d), dtype=wl.Kc.dtype)
    VP = torch.zeros_like(KP)
    table, items, e = [], [], 0
    for b, p in enumerate(P):
        items.append((b, 0, wl.q, e, p))
        for j in range(n_pages[b]):
            n = min(page, p - j * page)
            KP[e, :n], VP[e, :n] = wl.Kc[b, j * page:j * page + n], wl.Vc[b, j * page:j * page + n]
            table.append(e)
            e += 1
    items = torch.tensor(items, dtype=torch.int32)
    table = torch.tensor(table, dtype=torch.int32)
    kv_max = int(wl.o.max())
    lse = torch.empty((wl.B, wl.Hq, wl.q), device="cuda")
    out = run_gpu(bd, wl, KP, VP, items, table, kv_max, lse=lse)
    t = wl.t
    Kc, Vc = wl.Kc.cuda(), wl.Vc.cuda()
    lse_p = torch.empty_like(lse)
    out_p = bd.attn_packed(wl.Q.cuda(), Kc, Vc, wl.o.cuda(), kv_max, Kc[:, t:], Vc[:, t:], wl.bl,
                           wl.sm_scale, lse=lse_p)
    torch.cuda.synchronize()
    assert torch.equal(out, out_p) and torch.equal(lse, lse_p)


def test_query_block_items_any_order(bd):
    """One item per (row, 32-query block), dispatched in a random order;
    query ranges that do not start on the kernel's query tiles."""
    note("block table: one item per query block")
    wl = synth.serving_mix(seed=13, B=4, p_lo=200, p_hi=2500, W=4, sparse_above=10 ** 9)
    KP, VP, table, rows = paged(wl, 128, seed=3)
    items = [(b, s, s + wl.bl, off, n) for b, _, _, off, n in rows.tolist() for s in range(0, wl.q, wl.bl)]
    items.append((0, 96, 10 ** 6, rows[0, 3].item(), rows[0, 4].item()))   # q_end clamped to q
    items = [it for it in items if not (it[0] == 0 and it[1] == 96 and it[2] == 128)]
    perm = np.random.default_rng(4).permutation(len(items))
    items = torch.tensor([items[i] for i in perm], dtype=torch.int32)
    kv_max = int(wl.o.max())
    out = run_gpu(bd, wl, KP, VP, items, table, kv_max)
    ref, _ = oracle(wl, KP, VP, items, table)
    check_items(out, ref, items, wl.q, "query blocks")


def test_split_prefix(bd):
    """Few items over long key lists: the plan splits each item's keys into
    chunks and merges them (the combine reads the item list)."""
    note("block table: split prefix")
    wl = synth.serving_mix(seed=14, B=2, p_lo=5000, p_hi=8000, W=1, sparse_above=10 ** 9)
    KP, VP, table, items = paged(wl, 128, seed=5)
    items[0, 4] -= 5
    kv_max = int(wl.o.max())
    assert bd.attn_block_table_workspace_size(torch.bfloat16, wl.Hq, wl.Hkv, wl.d, wl.q,
                                              len(items), kv_max) > 0
    items = items.flip(0).contiguous()
    out = run_gpu(bd, wl, KP, VP, items, table, kv_max)
    ref, _ = oracle(wl, KP, VP, items, table)
    check_items(out, ref, items, wl.q, "split")


def test_items_added_and_removed(bd):
    """Two calls with different item lists on one output: rows the second
    call drops keep the first call's outputs; a row whose list shrank (its
    last two pages removed) and a newly added row match the oracle."""
    note("block table: items added and removed between calls")
    wl = synth.serving_mix(seed=15, B=5, p_lo=300, p_hi=3000, W=2, sparse_above=10 ** 9)
    KP, VP, table, items = paged(wl, 64, seed=6)
    kv_max = int(wl.o.max())
    first = items[[0, 1, 2]].contiguous()
    out = run_gpu(bd, wl, KP, VP, first, table, kv_max)
    keep = out.clone()
    second = items[[3, 1]].clone()
    second[1, 4] = max(0, int(second[1, 4]) - 2 * 64 - 17)
    out = run_gpu(bd, wl, KP, VP, second.contiguous(), table, kv_max, out=out)
    ref, _ = oracle(wl, KP, VP, second, table)
    check_attention(out[1:2], ref[1:2], torch.bfloat16, label="shrunk row")
    check_attention(out[3:4], ref[3:4], torch.bfloat16, label="added row")
    assert torch.equal(bits_t(out[[0, 2]]), bits_t(keep[[0, 2]]))
    assert (out[4].float() == SENTINEL).all()


def bits_t(x):
    return torch.from_numpy(bits(x))


def test_out_of_range_page_ids(bd):
    """Page ids outside [0, n_pages) contribute no keys: the result is the
    oracle's over the list without those pages."""
    note("block table: out-of-range page ids")
    wl = synth.serving_mix(seed=16, B=2, p_lo=1000, p_hi=2000, W=2, sparse_above=10 ** 9)
    page = 64
    KP, VP, table, items = paged(wl, page, seed=7)
    kv_max = int(wl.o.max())
    bad = table.clone()
    off0 = int(items[0, 3])
    bad[off0 + 1] = -5                       # full pages of row 0
    bad[off0 + 4] = KP.shape[0] + 3
    out = run_gpu(bd, wl, KP, VP, items, bad, kv_max)
    # the same keys without pages 1 and 4 of row 0
    keep = [j for j in range(len(table)) if j not in (off0 + 1, off0 + 4)]
    t2 = table[keep]
    it2 = items.clone()
    it2[0, 4] -= 2 * page
    it2[1, 3] -= 2
    ref, _ = oracle(wl, KP, VP, it2, t2)
    check_items(out, ref, items, wl.q, "bad page ids")
