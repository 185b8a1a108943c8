"""Float64 CPU oracle for block-diffusion attention over a KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
import this module.  The HIP library never calls it and shares no code
with it.

Every function is the plain definition written out in NumPy float64, one
(row, KV head) at a time, with no blocking, fusion or reordering beyond
what the definition states.  Inputs given in bf16 or fp32 convert to f64
exactly.  Sources (the pages the method is described on):

* HERALD: High-Throughput Block Diffusion LLM Serving via CPU-GPU
  Cooperative KV Cache Retrieval ("HERALD" below).
* FlowBlock: Wavefront-Parallel Decoding for Self-Correcting Diffusion
  Language Models, blog review ("FlowBlock review" below).  The review
  numbers its equations (1)-(7); the paper's own numbers are one lower
  from (3) on.  Both are given.

Readings taken where the pages leave a step open (each is repeated in the
design notes):

* softmax scale ``sm_scale`` is an explicit argument (1/sqrt(d) in every
  workload); the same value is used for selection and attention.
* GQA head map: query head ``hq`` reads KV head ``hq // G``.
* the representative query is either the mean of the block's queries or
  one given query row; ``center_row`` implements HERALD Eq. (2).
* selection scans prefix positions ``s < S_b`` only; top-k ties go to the
  lower position and the kept positions are returned in ascending order.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, a library routine (torch SDPA, scipy)
or the worked example printed on the FlowBlock review.  No function is
unpinned.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "eq6_mask",
    "window_visible",
    "block_attention",
    "block_table_attention",
    "cache_attention_eq6",
    "rep_query",
    "center_row",
    "selection_scores",
    "rep_attention",
    "multi_query_scores",
    "topk_select",
    "gather",
    "kv_scatter",
    "rope",
    "qkv_rope",
]


def _f64(x):
    """Exact conversion of a NumPy or torch (CPU) array to float64.  The
    functions below convert one (row, KV head) slice at a time, so inputs
    may be far larger than their float64 copy would be."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int64)


# ---------------------------------------------------------------------------
# Mask
# ---------------------------------------------------------------------------

MASK_MODES = ("block_causal", "isolated", "shared_first")


def eq6_mask(C: int, q: int, bl: int, o, mode: str = "block_causal") -> np.ndarray:
    """Per-row block-diagonal mask over a cache of capacity ``C``.

    FlowBlock review, Eq. (6) (paper Eq. 5): query ``i`` of row ``b`` sees
    key ``j`` when ``j < o_b`` (the row's own frozen prefix) or when
    ``t <= j < t + (s+1)*bl`` with ``t = C - q`` the shared physical tail
    where the window's present KV lives and ``s = floor(i / bl)`` the
    query's window slot.  Other ``mode`` values replace the tail part by
    ``window_visible``'s other modes (the prefix part is unchanged).

    Returns a bool array ``[B, q, C]``.
    """
    o = _i64(o)
    t = C - q
    j = np.arange(C)[None, :]
    own_tail = np.zeros((q, C), bool)
    own_tail[:, t:] = window_visible(q, bl, mode)          # [q, C]
    own_prefix = j[None, :, :] < o[:, None, None]          # [B, 1, C]
    return own_prefix | own_tail[None, :, :]


def window_visible(q: int, bl: int, mode: str = "block_causal") -> np.ndarray:
    """Window part of the mask in window coordinates ``w = j - t``; the
    window holds ``q / bl`` blocks (groups) of ``bl`` queries and keys.

    ``block_causal`` (FlowBlock review Eq. (6)): query ``i`` sees window key
    ``w`` when ``w < (floor(i/bl) + 1) * bl``: bidirectional inside its own
    block and causal over earlier window blocks (W-shaped mask).

    ``isolated`` (HERALD Sec. IV-B2): the denoising group and the draft
    group run in one forward pass; each sees the prefix and its own group
    (bidirectionally) but not the other: ``floor(w/bl) == floor(i/bl)``.

    ``shared_first`` (Flash-dLLM's verify pass; reading of a garbled
    passage): block 0 holds the tracked context, the later blocks are views
    of the search positions; the context does not see the views and the
    views do not see each other, each view sees the context:
    ``floor(w/bl) == floor(i/bl)`` or ``floor(w/bl) == 0``.

    Returns ``[q, q]`` bool.
    """
    if mode not in MASK_MODES:
        raise ValueError(f"unknown mask mode {mode!r}")
    gi = np.arange(q)[:, None] // bl
    gw = np.arange(q)[None, :] // bl
    if mode == "block_causal":
        return gw <= gi
    if mode == "isolated":
        return gw == gi
    return (gw == gi) | (gw == 0)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _softmax_attend(logits: np.ndarray, vals: np.ndarray):
    """Softmax over the last axis of ``logits`` then weighted sum of ``vals``.

    ``logits`` holds -inf where a key is not visible.  Returns (out, lse)
    with ``lse = m + log(sum exp(logits - m))`` (FlashAttention statistics,
    HERALD Sec. IV-B4).
    """
    m = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - m)
    z = p.sum(axis=-1, keepdims=True)
    out = (p @ vals) / z
    lse = (m + np.log(z))[..., 0]
    return out, lse


def block_attention(Q, PK, PV, p_len, WK, WV, bl: int, sm_scale: float,
                    rows=None, mode: str = "block_causal"):
    """Block-diffusion attention in prefix/window form.

    For row ``b``, query ``i`` and query head ``hq`` (KV head ``h = hq//G``)
    the visible keys are every prefix entry ``PK[b, 0:p_len[b], h]`` and the
    window entries ``WK[b, w, h]`` with ``w < (floor(i/bl)+1)*bl``.  With
    ``PK`` the cache and ``p_len = o`` this is FlowBlock review Eq. (6)
    (the window is the cache tail ``[t, C)``); with ``PK`` a compact pool of
    selected entries and ``p_len = k_b`` it is HERALD's denoising attention
    over the critical KV cache (Sec. III-C, IV-B1), where the block attends
    bidirectionally in-block and to the cached prefix (Sec. II-A).  ``mode``
    picks the window mask (``window_visible``).

    Q: [B, q, Hq, d]; PK, PV: [B, P, Hkv, d]; WK, WV: [B, q, Hkv, d].
    Returns ``O [B, q, Hq, d]`` and ``LSE [B, Hq, q]`` in float64; rows not
    in ``rows`` are NaN.
    """
    Q = _f64(Q)
    p_len = _i64(p_len)
    B, q, Hq, d = Q.shape
    Hkv = PK.shape[2]
    G = Hq // Hkv
    assert G * Hkv == Hq
    rows = range(B) if rows is None else [int(r) for r in _i64(rows)]
    wvis = window_visible(q, bl, mode)                       # [q, q]
    O = np.full((B, q, Hq, d), np.nan)
    LSE = np.full((B, Hq, q), np.nan)
    for b in rows:
        P = int(p_len[b])
        for h in range(Hkv):
            keys = np.concatenate([_f64(PK[b, :P, h]), _f64(WK[b, :, h])], axis=0)
            vals = np.concatenate([_f64(PV[b, :P, h]), _f64(WV[b, :, h])], axis=0)
            vis = np.concatenate([np.ones((q, P), bool), wvis], axis=1)
            for g in range(G):
                hq = h * G + g
                logits = sm_scale * (Q[b, :, hq] @ keys.T)   # [q, P+q]
                logits = np.where(vis, logits, -np.inf)
                O[b, :, hq], LSE[b, hq] = _softmax_attend(logits, vals)
    return O, LSE


def block_table_attention(Q, KP, VP, items, table, page: int, WK, WV, bl: int,
                          sm_scale: float, kv_max: int | None = None):
    """Attention scheduled by a block table (Flash-dLLM, Scheduled Flash
    Attention, Fig. 3(b)).

    The batch is cut into work items; the block table aligns each item's
    query block with the key-value blocks it attends over.  Here the
    key-value blocks are pages of a paged store ``KP, VP [n_pages, page, Hkv,
    d]``.  Item ``(row, q_begin, q_end, table_off, kv_len)`` covers queries
    ``i`` in ``[q_begin, min(q_end, q))`` of ``row``; its keys are the first
    ``L = min(kv_len, kv_max)`` keys of the pages ``table[table_off + j]``
    taken in table order (key ``m`` is position ``m % page`` of page
    ``table[table_off + m // page]``), followed by the row's window keys
    ``WK[row, w]`` with ``w < (floor(i/bl) + 1) * bl`` (FlowBlock review
    Eq. (6)'s window part).  A contiguous table over a row's own cache is
    ``block_attention`` with ``p_len = kv_len``.

    Q: [B, q, Hq, d]; WK, WV: [B, q, Hkv, d]; items: int array [n, 5];
    table: int array.  Returns ``O [B, q, Hq, d]`` and ``LSE [B, Hq, q]`` in
    float64, NaN wherever no item writes.
    """
    Q = _f64(Q)
    items = _i64(items).reshape(-1, 5)
    table = _i64(table)
    B, q, Hq, d = Q.shape
    Hkv = KP.shape[2]
    G = Hq // Hkv
    wvis = window_visible(q, bl)                              # [q, q]
    O = np.full((B, q, Hq, d), np.nan)
    LSE = np.full((B, Hq, q), np.nan)
    for row, q0, q1, off, n in items:
        q1 = min(int(q1), q)
        L = int(n) if kv_max is None else min(int(n), int(kv_max))
        pages = table[int(off):int(off) + -(-L // page)]
        qi = np.arange(int(q0), q1)
        for h in range(Hkv):
            pk = np.concatenate([_f64(KP[p, :, h]) for p in pages] + [np.zeros((0, d))])[:L]
            pv = np.concatenate([_f64(VP[p, :, h]) for p in pages] + [np.zeros((0, d))])[:L]
            keys = np.concatenate([pk, _f64(WK[row, :, h])], axis=0)
            vals = np.concatenate([pv, _f64(WV[row, :, h])], axis=0)
            vis = np.concatenate([np.ones((len(qi), L), bool), wvis[qi]], axis=1)
            for g in range(G):
                hq = h * G + g
                logits = sm_scale * (Q[row, qi, hq] @ keys.T)
                logits = np.where(vis, logits, -np.inf)
                O[row, qi, hq], LSE[row, hq, qi] = _softmax_attend(logits, vals)
    return O, LSE


def cache_attention_eq6(Q, Kc, Vc, o, bl: int, sm_scale: float, mode: str = "block_causal"):
    """Attention over the whole pre-allocated cache under the Eq. (6) mask.

    FlowBlock review Eq. (6): the keys are the cache positions ``j`` of
    ``[0, C)`` that ``eq6_mask`` marks visible; all other positions are
    never read (they may hold anything, NaN included).  Kc, Vc:
    ``[B, C, Hkv, d]``.  Returns ``O [B, q, Hq, d]``, ``LSE [B, Hq, q]``.
    """
    Q = _f64(Q)
    B, q, Hq, d = Q.shape
    C, Hkv = Kc.shape[1], Kc.shape[2]
    G = Hq // Hkv
    M = eq6_mask(C, q, bl, o, mode)
    O = np.empty((B, q, Hq, d))
    LSE = np.empty((B, Hq, q))
    for b in range(B):
        cols = np.nonzero(M[b].any(axis=0))[0]             # keys read at all
        vis = M[b][:, cols]
        for h in range(Hkv):
            keys, vals = _f64(Kc[b, cols, h]), _f64(Vc[b, cols, h])
            for g in range(G):
                hq = h * G + g
                logits = sm_scale * (Q[b, :, hq] @ keys.T)
                logits = np.where(vis, logits, -np.inf)
                O[b, :, hq], LSE[b, hq] = _softmax_attend(logits, vals)
    return O, LSE


# ---------------------------------------------------------------------------
# Representative query and selection scores
# ---------------------------------------------------------------------------

def center_row(bl: int, S: int) -> int:
    """Block position HERALD Eq. (2) picks as the representative query.

    Eq. (2): the position ``p_i`` of the block minimising
    ``sum_s (p_i - s - mean_offset)^2`` over prefix positions ``s``.  For an
    even block the two middle positions tie exactly; the page speaks of the
    block centre with offsets of at most ``B/2`` from it, and the later of
    the two (``bl // 2``) is taken.
    """
    o = S  # block starts right after the prefix; the result is shift-free
    pos = o + np.arange(bl, dtype=np.float64)
    s = np.arange(S, dtype=np.float64)
    mean_off = (pos[:, None] - s[None, :]).mean()
    obj = ((pos[:, None] - s[None, :] - mean_off) ** 2).sum(axis=1)
    best = obj.min()
    ties = np.nonzero(np.isclose(obj, best, rtol=1e-12, atol=0.0))[0]
    return int(ties.max())


def rep_query(Q, mode: str = "mean", row: int | None = None):
    """Representative query per (row, query head), float64 ``[B, Hq, d]``.

    HERALD Sec. IV-A2 replaces the block's queries by one representative.
    ``mode='row'`` takes query ``row`` of the block (HERALD's choice is the
    centre, see ``center_row``); ``mode='mean'`` averages the ``nq`` queries
    given (the sparse workloads use the mean of the block's queries).
    Q: ``[B, nq, Hq, d]``.
    """
    Q = _f64(Q)
    if mode == "mean":
        return Q.mean(axis=1)
    if mode == "row":
        return Q[:, int(row)].copy()
    raise ValueError(mode)


def selection_scores(q_rep, K, s_len, sm_scale: float):
    """GQA importance of every prefix position, HERALD Sec. IV-B4.

    For row ``b`` and KV head ``h`` with query heads ``g < G``:
    ``z[g, s] = sm_scale * <q_rep[b, h*G+g], K[b, s, h]>`` for ``s < S_b``,
    ``m_g = max_s z[g, s]``, ``l_g = sum_s exp(z[g, s] - m_g)`` and
    ``s_hat[s] = sum_g exp(z[g, s] - m_g) / l_g``.

    q_rep: ``[B, Hq, d]``; K: ``[B, C, Hkv, d]``; s_len: ``[B]``.
    Returns ``s_hat [B, Hkv, max(s_len)]`` (0 past ``S_b``), ``m`` and ``l``
    ``[B, Hq]`` (NaN for rows with ``S_b = 0``).
    """
    q_rep = _f64(q_rep)
    s_len = _i64(s_len)
    B, Hq, d = q_rep.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    s_max = int(s_len.max()) if len(s_len) else 0
    s_hat = np.zeros((B, Hkv, s_max))
    m = np.full((B, Hq), np.nan)
    l = np.full((B, Hq), np.nan)
    for b in range(B):
        S = int(s_len[b])
        if S == 0:
            continue
        for h in range(Hkv):
            qg = q_rep[b, h * G:(h + 1) * G]               # [G, d]
            z = sm_scale * (qg @ _f64(K[b, :S, h]).T)      # [G, S]
            mg = z.max(axis=1, keepdims=True)
            e = np.exp(z - mg)
            lg = e.sum(axis=1, keepdims=True)
            s_hat[b, h, :S] = (e / lg).sum(axis=0)
            m[b, h * G:(h + 1) * G] = mg[:, 0]
            l[b, h * G:(h + 1) * G] = lg[:, 0]
    return s_hat, m, l


def rep_attention(q_rep, K, V, s_len, sm_scale: float):
    """Attention output of the representative query over the full prefix,
    HERALD Sec. IV-B4: beside the scores, the fused selection kernel keeps
    the running output ``o_g`` of every query head with ``(m_g, l_g)``, and
    the output goes back at once so the next layer's FFN can run.

    For row ``b`` and query head ``hq = h*G + g`` (KV head ``h``):
    ``o[b, hq] = sum_s exp(z[g, s] - m_g) / l_g * V[b, s, h]`` over
    ``s < S_b``, with ``z``, ``m_g``, ``l_g`` as in ``selection_scores``:
    single-query softmax attention over the prefix.  Rows with ``S_b = 0``
    have no output (zeros).

    q_rep: ``[B, Hq, d]``; K, V: ``[B, C, Hkv, d]``; s_len: ``[B]``.
    Returns ``o [B, Hq, d]`` float64.
    """
    q_rep = _f64(q_rep)
    s_len = _i64(s_len)
    B, Hq, d = q_rep.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Hq, d))
    for b in range(B):
        S = int(s_len[b])
        if S == 0:
            continue
        for h in range(Hkv):
            qg = q_rep[b, h * G:(h + 1) * G]               # [G, d]
            z = sm_scale * (qg @ _f64(K[b, :S, h]).T)      # [G, S]
            o[b, h * G:(h + 1) * G], _ = _softmax_attend(z, _f64(V[b, :S, h]))
    return o


def multi_query_scores(Q, K, s_len, sm_scale: float):
    """Exact multi-query importance: every block query ranks the prefix.

    HERALD Sec. III-C and Sec. IV-A2: before the query reduction, the
    selection phase runs exact attention of all of the block's queries over
    the full prefix KV (MAGE's selection at a block's first step; the
    queries form a GEMM), and Fig. 8 sweeps the number of queries used.
    The per-query probabilities are aggregated the way Sec. IV-B4 aggregates
    the G query heads of a KV head: summed.  For row ``b``, KV head ``h``,
    query ``i < nq`` and group head ``g < G``:
    ``z[i, g, s] = sm_scale * <Q[b, i, h*G+g], K[b, s, h]>`` for ``s < S_b``
    and ``s_hat[s] = sum_i sum_g exp(z[i, g, s] - m_ig) / l_ig`` with
    ``m_ig = max_s z[i, g, s]``, ``l_ig = sum_s exp(z[i, g, s] - m_ig)``.
    With ``nq = 1`` this is ``selection_scores`` with that query as q_rep.

    Q: ``[B, nq, Hq, d]``; K: ``[B, C, Hkv, d]``; s_len: ``[B]``.
    Returns ``s_hat [B, Hkv, max(s_len)]`` (0 past ``S_b``).
    """
    s_len = _i64(s_len)
    B, nq, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    s_max = int(s_len.max()) if len(s_len) else 0
    s_hat = np.zeros((B, Hkv, s_max))
    for b in range(B):
        S = int(s_len[b])
        if S == 0:
            continue
        Qb = _f64(Q[b])                                    # [nq, Hq, d]
        for h in range(Hkv):
            cols = Qb[:, h * G:(h + 1) * G].reshape(nq * G, d)   # rows (i, g)
            z = sm_scale * (cols @ _f64(K[b, :S, h]).T)          # [nq*G, S]
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            s_hat[b, h, :S] = (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
    return s_hat


def topk_select(scores, s_len, k_sel, k_max: int) -> np.ndarray:
    """Per-(row, KV head) top-k critical set, HERALD Sec. IV-B4.

    Keeps the ``min(k_b, S_b)`` positions with the largest score; equal
    scores go to the lower position.  The kept positions are written in
    ascending order and the rest of the ``k_max`` slots hold -1.
    scores: ``[B, Hkv, >= S_b]``.  Returns int64 ``[B, Hkv, k_max]``.
    """
    scores = _f64(scores)
    s_len, k_sel = _i64(s_len), _i64(k_sel)
    B, Hkv = scores.shape[:2]
    out = np.full((B, Hkv, k_max), -1, dtype=np.int64)
    for b in range(B):
        S = int(s_len[b])
        k = min(int(k_sel[b]), S)
        if k <= 0:
            continue
        for h in range(Hkv):
            sc = scores[b, h, :S]
            order = np.lexsort((np.arange(S), -sc))        # score desc, pos asc
            out[b, h, :k] = np.sort(order[:k])
    return out


# ---------------------------------------------------------------------------
# KV movement
# ---------------------------------------------------------------------------

def gather(src, idx, k_cnt, pool):
    """Copy selected entries into the compact pool, HERALD Sec. IV-B3.

    ``pool[b, j, h] = src[b, idx[b, h, j], h]`` for ``j < k_cnt[b]``; every
    other pool slot keeps its value.  Works on any dtype (bit copy).
    """
    src = np.asarray(src)
    pool = np.array(pool, copy=True)
    idx, k_cnt = _i64(idx), _i64(k_cnt)
    B, Hkv = idx.shape[:2]
    for b in range(B):
        for h in range(Hkv):
            for j in range(int(k_cnt[b])):
                pool[b, j, h] = src[b, idx[b, h, j], h]
    return pool


def kv_scatter(present, data, o, t: int, q: int, rows=None):
    """KV write-back, FlowBlock review Eq. (7) (paper Eq. 6).

    ``data[l, b, o_b + delta] <- present[l, b, t + delta]`` for
    ``delta < q`` and every layer ``l``; everything else in ``data`` keeps
    its value.  present, data: ``[L, B, P, Hkv, d]`` (any dtype, bit copy).
    ``present`` may be the same array as ``data``; the source rows are read
    before any write.
    """
    present = np.asarray(present)
    src = present[:, :, t:t + q].copy()
    data = np.array(data, copy=True)
    o = _i64(o)
    B = data.shape[1]
    rows = range(B) if rows is None else [int(r) for r in _i64(rows)]
    for b in rows:
        ob = int(o[b])
        data[:, b, ob:ob + q] = src[:, b]
    return data


# ---------------------------------------------------------------------------
# Fused producer: QKV projection, rotary embedding, cache write
# ---------------------------------------------------------------------------

def rope(x, pos, base: float = 10000.0):
    """Rotary positional embedding of head vectors at absolute positions.

    HERALD Eq. (1) writes the rotation R_{theta,p} applied to a query or key
    at position p; FlowBlock's packed windows use absolute positions.  The
    pages fix neither the frequencies nor the pairing; the reading is the
    usual one: dimension j < d/2 pairs with j + d/2 and turns by the angle
    ``p * base**(-2j/d)``.  x: ``[..., n, d]`` with ``pos`` ``[n]``.
    """
    x = _f64(x)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * base ** (-2.0 * np.arange(h) / d)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def qkv_rope(X, Wqkv, rope_pos, Hq: int, Hkv: int, base: float = 10000.0):
    """Flash-dLLM's fused cache producer (Flash-Cache): the projection of the
    window's hidden states, RoPE on queries and keys, and the keys and values
    that the cache write stores.

    X: ``[B, q, Dm]``; Wqkv: ``[(Hq + 2*Hkv) * d, Dm]`` (rows: the query heads,
    then the key heads, then the value heads); window token ``i`` of row ``b``
    sits at absolute position ``rope_pos[b] + i``.  Returns Q ``[B, q, Hq, d]``,
    K and V ``[B, q, Hkv, d]`` in float64.
    """
    X = _f64(X)
    W = _f64(Wqkv)
    rope_pos = _i64(rope_pos)
    B, q, Dm = X.shape
    d = W.shape[0] // (Hq + 2 * Hkv)
    Q = np.empty((B, q, Hq, d))
    K = np.empty((B, q, Hkv, d))
    V = np.empty((B, q, Hkv, d))
    for b in range(B):
        Y = (X[b] @ W.T).reshape(q, Hq + 2 * Hkv, d)          # [q, heads, d]
        pos = int(rope_pos[b]) + np.arange(q)
        Q[b] = np.stack([rope(Y[:, hq], pos, base) for hq in range(Hq)], axis=1)
        K[b] = np.stack([rope(Y[:, Hq + h], pos, base) for h in range(Hkv)], axis=1)
        V[b] = Y[:, Hq + Hkv:]
    return Q, K, V
