"""Pins of the oracle's block-table attention (Flash-dLLM, Scheduled Flash
Attention, Fig. 3(b)): a block table aligns each work item's query block
with the key-value blocks (pages) it attends over.

- a contiguous table over a row's own cache equals the prefix/window form
  of FlowBlock review Eq. (6) (``block_attention``, itself pinned to torch
  SDPA), including a ragged last page and an empty key list;
- the physical placement of the pages does not matter (shuffled store,
  remapped table: identical result);
- the order of the pages in the table does not change the result beyond
  rounding (softmax over a set of keys);
- splitting a row's queries over several items gives the same outputs;
- one item against torch SDPA in float64 with an explicit boolean mask;
- outputs no item covers stay untouched (NaN).
"""
import math

import numpy as np
import pytest
import torch

from oracle import bd_oracle as orc

B, q, bl, Hq, Hkv, d, page = 3, 64, 32, 4, 2, 16, 8


def _data(seed=0, P=(40, 61, 0)):
    """A row cache [B, C, Hkv, d] with the window at its tail, and the same
    prefixes cut into pages of a paged store in row order."""
    g = np.random.default_rng(seed)
    C = max(P) + q + 8
    Kc = g.standard_normal((B, C, Hkv, d))
    Vc = g.standard_normal((B, C, Hkv, d))
    Q = g.standard_normal((B, q, Hq, d))
    t = C - q
    n_pages = [math.ceil(p / page) for p in P]
    KP = np.zeros((sum(n_pages), page, Hkv, d))
    VP = np.zeros_like(KP)
    table, items, e = [], [], 0
    for b, p in enumerate(P):
        off = len(table)
        for j in range(n_pages[b]):
            n = min(page, p - j * page)
            KP[e, :n] = Kc[b, j * page:j * page + n]
            VP[e, :n] = Vc[b, j * page:j * page + n]
            table.append(e)
            e += 1
        items.append((b, 0, q, off, p))
    return dict(Kc=Kc, Vc=Vc, Q=Q, t=t, P=np.array(P), KP=KP, VP=VP,
                table=np.array(table), items=np.array(items))


def _bt(x, items=None, table=None, KP=None, VP=None):
    return orc.block_table_attention(x["Q"], x["KP"] if KP is None else KP,
                                     x["VP"] if VP is None else VP,
                                     x["items"] if items is None else items,
                                     x["table"] if table is None else table, page,
                                     x["Kc"][:, x["t"]:], x["Vc"][:, x["t"]:], bl, 0.3)


def test_contiguous_table_is_block_attention():
    x = _data()
    O, L = _bt(x)
    Or, Lr = orc.block_attention(x["Q"], x["Kc"], x["Vc"], x["P"], x["Kc"][:, x["t"]:],
                                 x["Vc"][:, x["t"]:], bl, 0.3)
    np.testing.assert_allclose(O, Or, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L, Lr, rtol=1e-13, atol=1e-13)
    assert np.isfinite(O).all()


def test_physical_page_placement_is_irrelevant():
    x = _data(1)
    perm = np.random.default_rng(5).permutation(len(x["KP"]))   # new slot of old page
    KP2 = np.empty_like(x["KP"])
    VP2 = np.empty_like(x["VP"])
    KP2[perm] = x["KP"]
    VP2[perm] = x["VP"]
    O1, L1 = _bt(x)
    O2, L2 = _bt(x, table=perm[x["table"]], KP=KP2, VP=VP2)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_page_order_in_the_table():
    """Full pages listed in another order: the same key set, the same
    softmax (rounding aside).  Row 0's 40 keys are 5 full pages."""
    x = _data(2, P=(40, 24, 16))
    items = x["items"].copy()
    table = x["table"].copy()
    off, n = items[0, 3], items[0, 4] // page
    table[off:off + n] = table[off:off + n][::-1]
    O1, L1 = _bt(x)
    O2, L2 = _bt(x, items=items, table=table)
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L2, L1, rtol=1e-12, atol=1e-12)


def test_queries_split_over_items():
    x = _data(3)
    split = []
    for b, q0, q1, off, n in x["items"]:
        for s in range(q0, q1, bl):
            split.append((b, s, min(s + bl, q1), off, n))
    split = np.array(split)[::-1]           # any dispatch order
    O1, L1 = _bt(x)
    O2, L2 = _bt(x, items=split)
    np.testing.assert_allclose(O2, O1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L2, L1, rtol=1e-13, atol=1e-13)


def test_one_item_against_sdpa():
    """Row 1, queries [32, 64): its 61 paged keys plus window keys < 64."""
    x = _data(4)
    b, q0, q1 = 1, 32, 64
    items = np.array([(b, q0, q1, x["items"][b, 3], x["items"][b, 4])])
    O, L = _bt(x, items=items)
    P = int(x["P"][b])
    t = x["t"]
    G = Hq // Hkv
    for h in range(Hkv):
        keys = np.concatenate([x["Kc"][b, :P, h], x["Kc"][b, t:, h]])
        vals = np.concatenate([x["Vc"][b, :P, h], x["Vc"][b, t:, h]])
        mask = np.zeros((q1 - q0, P + q), bool)
        mask[:, :P] = True
        mask[:, P:P + 64] = True                 # queries 32..63: window keys < 64
        for g in range(G):
            hq = h * G + g
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(x["Q"][b, q0:q1, hq])[None, None],
                torch.from_numpy(keys)[None, None], torch.from_numpy(vals)[None, None],
                attn_mask=torch.from_numpy(mask)[None, None], scale=0.3)[0, 0].numpy()
            np.testing.assert_allclose(O[b, q0:q1, hq], ref, rtol=1e-12, atol=1e-12)
    # nothing else written
    assert np.isnan(O[b, :q0]).all() and np.isnan(O[0]).all() and np.isnan(O[2]).all()
    assert np.isnan(L[b, :, :q0]).all()


def test_window_only_and_kv_max():
    """kv_len 0 (row 2) is the window alone; kv_max truncates every list."""
    x = _data(5)
    O, _ = _bt(x)
    Or, _ = orc.block_attention(x["Q"], x["Kc"], x["Vc"], np.zeros(B, int), x["Kc"][:, x["t"]:],
                                x["Vc"][:, x["t"]:], bl, 0.3)
    np.testing.assert_allclose(O[2], Or[2], rtol=1e-13, atol=1e-13)
    O3, _ = orc.block_table_attention(x["Q"], x["KP"], x["VP"], x["items"], x["table"], page,
                                      x["Kc"][:, x["t"]:], x["Vc"][:, x["t"]:], bl, 0.3, kv_max=20)
    Or3, _ = orc.block_attention(x["Q"], x["Kc"], x["Vc"], np.minimum(x["P"], 20),
                                 x["Kc"][:, x["t"]:], x["Vc"][:, x["t"]:], bl, 0.3)
    np.testing.assert_allclose(O3, Or3, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("bad", ["order", "offset", "window"])
def test_pins_catch_planted_mistakes(bad, monkeypatch):
    """Each pin above fails on a plausible mistake planted in the oracle:
    pages in reverse order inside a row, keys read one position late within
    a page, or the window mask of the next block."""
    x = _data(6)
    Or, _ = orc.block_attention(x["Q"], x["Kc"], x["Vc"], x["P"], x["Kc"][:, x["t"]:],
                                x["Vc"][:, x["t"]:], bl, 0.3)
    KP, VP, table, items = x["KP"], x["VP"], x["table"], x["items"]
    WK, WV = x["Kc"][:, x["t"]:], x["Vc"][:, x["t"]:]
    if bad == "order":
        table = table.copy()
        table[items[1, 3]:items[1, 3] + 8] = table[items[1, 3]:items[1, 3] + 8][::-1]
        # a ragged last page moved first changes which keys are counted
    elif bad == "offset":
        KP = np.roll(KP, 1, axis=1)
    else:
        monkeypatch.setattr(orc, "window_visible",
                            lambda q_, bl_, mode="block_causal": (np.arange(q_)[None, :] // bl_)
                            <= (np.arange(q_)[:, None] // bl_ + 1))
    O, _ = orc.block_table_attention(x["Q"], KP, VP, items, table, page, WK, WV, bl, 0.3)
    assert not np.allclose(O, Or, rtol=1e-6, atol=1e-6)
