"""One step of the block-diffusion hot path over a batch of packed rows.

Holds the device buffers allocated once at set-up (pools, indices, scores,
outputs, workspaces; HERALD Sec. V allocates its pools at initialisation
and reuses them) and issues the library calls of one step in order:

  1. bd_select over the sparse rows (representative query + top-k),
  2. bd_gather of the selected K/V into the pool,
  3. one bd_attn_packed_dual launch: the dense rows over their own cache,
     the sparse rows over their pools (the short pool rows fill the tail of
     the long cache rows); bd_attn_packed when only one kind is present,
  4. bd_kv_scatter of every row's window to its absolute position.

attn_dense / attn_sparse run the two row kinds as separate launches (the
same results; used to time them one by one).

Every step runs in the HIP kernels on the current stream; this class only
marshals arguments.  Repeated steps are idempotent: the scatter writes the
window into [o_b, o_b + q), which neither the selection (positions < o_b)
nor the attention (prefix < o_b, window at the tail) reads.
"""
from __future__ import annotations

import torch

from . import bdattn as bd


class BlockDiffusionStep:
    def __init__(self, Kc, Vc, Q, o, bl: int, sm_scale: float, sparse_rows=None, dense_rows=None,
                 s_len=None, k_sel=None, p_max_dense: int | None = None, k_max: int = 0,
                 s_max: int = 0, n_layers: int = 1):
        self.dev = Kc.device
        self.Kc, self.Vc, self.Q, self.o = Kc, Vc, Q, o
        self.B, self.C, self.Hkv, self.d = Kc.shape
        self.Hq = Q.shape[2]
        self.q = Q.shape[1]
        self.t = self.C - self.q
        self.bl = bl
        self.sm_scale = sm_scale
        self.wk, self.wv = Kc[:, self.t:], Vc[:, self.t:]
        B = self.B
        i32 = dict(dtype=torch.int32, device=self.dev)
        self.sparse_rows = (sparse_rows.to(self.dev) if sparse_rows is not None
                            else torch.zeros(0, **i32))
        self.dense_rows = (dense_rows.to(self.dev) if dense_rows is not None
                           else torch.arange(B, **i32))
        self.n_sparse = int(self.sparse_rows.numel())
        self.n_dense = int(self.dense_rows.numel())
        self.p_max_dense = int(p_max_dense) if p_max_dense is not None else self.C - self.q
        self.k_max = int(k_max)
        self.s_max = int(s_max)
        self.s_len = s_len.to(self.dev) if s_len is not None else torch.zeros(B, **i32)
        self.k_sel = k_sel.to(self.dev) if k_sel is not None else torch.zeros(B, **i32)
        # entries a row's pool holds: bd_select keeps min(k_b, S_b) positions
        # (-1 past them), so a budget above the prefix fills only S_b slots
        self.k_eff = torch.minimum(self.k_sel, self.s_len).contiguous()
        self.out = torch.zeros_like(Q)
        if self.n_sparse:
            self.idx = torch.empty((B, self.Hkv, self.k_max), **i32)
            self.scores = torch.empty((B, self.Hkv, self.s_max), dtype=torch.float32, device=self.dev)
            self.pool_k = torch.zeros((B, self.k_max, self.Hkv, self.d), dtype=Kc.dtype, device=self.dev)
            self.pool_v = torch.zeros_like(self.pool_k)
            self.ws_sel = bd.workspace(bd.select_workspace_size(B, self.Hq, self.Hkv, self.d,
                                                                self.s_max, self.k_max), self.dev)
            self.ws_sparse = bd.workspace(bd.attn_workspace_size(
                Q.dtype, B, self.Hq, self.Hkv, self.d, self.q, self.n_sparse, self.k_max), self.dev)
        if self.n_dense:
            self.ws_dense = bd.workspace(bd.attn_workspace_size(
                Q.dtype, B, self.Hq, self.Hkv, self.d, self.q, self.n_dense, self.p_max_dense),
                self.dev)
        if self.n_dense and self.n_sparse:
            self.ws_both = bd.workspace(bd.attn_dual_workspace_size(
                Q.dtype, B, self.Hq, self.Hkv, self.d, self.q, self.n_dense, self.p_max_dense,
                self.n_sparse, self.k_max), self.dev)

    # individual ops (so callers can time them one by one)
    def select(self):
        if self.n_sparse:
            bd.select(self.Q, self.Kc, self.s_len, self.s_max, self.k_sel, self.k_max,
                      self.sm_scale, idx_out=self.idx, score_out=self.scores, ws=self.ws_sel)

    def gather(self):
        if self.n_sparse:
            bd.gather(self.Kc, self.Vc, self.idx, self.k_eff, self.pool_k, self.pool_v)

    def attn_dense(self):
        if self.n_dense:
            bd.attn_packed(self.Q, self.Kc, self.Vc, self.o, self.p_max_dense, self.wk, self.wv,
                           self.bl, self.sm_scale, out=self.out, row_ids=self.dense_rows,
                           ws=self.ws_dense)

    def attn_sparse(self):
        if self.n_sparse:
            bd.attn_packed(self.Q, self.pool_k, self.pool_v, self.k_eff, self.k_max, self.wk,
                           self.wv, self.bl, self.sm_scale, out=self.out,
                           row_ids=self.sparse_rows, ws=self.ws_sparse)

    def attn(self):
        """Attention of every row in one launch."""
        if self.n_dense and self.n_sparse:
            bd.attn_packed_dual(self.Q, (self.dense_rows, self.Kc, self.Vc, self.o, self.p_max_dense),
                                (self.sparse_rows, self.pool_k, self.pool_v, self.k_eff, self.k_max),
                                self.wk, self.wv, self.bl, self.sm_scale, out=self.out,
                                ws=self.ws_both)
        else:
            self.attn_dense()
            self.attn_sparse()

    def scatter(self):
        bd.kv_scatter(self.Kc, self.Vc, self.Kc, self.Vc, self.o, self.t, self.q)

    OPS = ("select", "gather", "attn", "scatter")

    def run(self):
        self.select()
        self.gather()
        self.attn()
        self.scatter()
        return self.out


class SparseBlockPipeline:
    """HERALD's dual-stream schedule of the sparse path on one GPU (Sec.
    IV-B2, Fig. 10; double-buffered sparse pools of Sec. IV-B1).

    Block n denoises for T steps on the main stream, each step one
    bd_attn_packed over pool[n % 2] plus that step's in-block KV.  Block
    n+1's selection phase (bd_select + bd_gather into pool[(n+1) % 2]) runs
    on a second stream: it starts once block n's second step has been issued
    (HERALD's draft of block n exists from then on) and block n+1's first
    step waits for its gather.  The pool a selection writes was last read by
    block n-1, which the main stream finished before block n's second step.

    ``run_sequential`` issues the same calls in order on one stream; both
    give bit-identical pools and outputs (the same kernels on the same
    inputs).  The selection inputs are the same for every block: the
    schedule, not the content of successive blocks, is what this measures.
    Both streams have the default priority.
    """

    def __init__(self, Kc, Vc, Qsel, s_len, k_sel, s_max: int, k_max: int, sm_scale: float,
                 bl: int, steps_q, steps_kv):
        self.dev = Kc.device
        self.Kc, self.Vc, self.Qsel = Kc, Vc, Qsel
        self.B, _, self.Hkv, self.d = Kc.shape
        self.Hq = Qsel.shape[2]
        self.s_len, self.k_sel = s_len, k_sel
        # pool entries per row: min(k_b, S_b) (bd_select pads the rest with -1)
        self.k_eff = torch.minimum(k_sel, s_len).contiguous()
        self.s_max, self.k_max = int(s_max), int(k_max)
        self.sm_scale, self.bl = sm_scale, bl
        self.steps_q, self.steps_kv = steps_q, steps_kv
        self.T = len(steps_q)
        i32 = dict(dtype=torch.int32, device=self.dev)
        self.idx = torch.empty((self.B, self.Hkv, self.k_max), **i32)
        self.pools = [(torch.zeros((self.B, self.k_max, self.Hkv, self.d), dtype=Kc.dtype,
                                   device=self.dev),
                       torch.zeros((self.B, self.k_max, self.Hkv, self.d), dtype=Kc.dtype,
                                   device=self.dev)) for _ in range(2)]
        self.out = torch.zeros_like(steps_q[0])
        nq = steps_q[0].shape[1]
        self.ws_sel = bd.workspace(bd.select_workspace_size(self.B, self.Hq, self.Hkv, self.d,
                                                            self.s_max, self.k_max), self.dev)
        self.ws_attn = bd.workspace(bd.attn_workspace_size(steps_q[0].dtype, self.B, self.Hq,
                                                           self.Hkv, self.d, nq, self.B,
                                                           self.k_max), self.dev)
        self.retrieval = torch.cuda.Stream(device=self.dev)
        self.ev_ready = [torch.cuda.Event(), torch.cuda.Event()]
        self.ev_draft = torch.cuda.Event()

    def retrieve(self, slot: int):
        """Selection phase of one block into pool ``slot`` (current stream)."""
        pk, pv = self.pools[slot]
        bd.select(self.Qsel, self.Kc, self.s_len, self.s_max, self.k_sel, self.k_max,
                  self.sm_scale, idx_out=self.idx, ws=self.ws_sel)
        bd.gather(self.Kc, self.Vc, self.idx, self.k_eff, pk, pv)

    def denoise(self, slot: int, st: int):
        """Denoising step ``st`` of one block over pool ``slot`` (current stream)."""
        pk, pv = self.pools[slot]
        wk, wv = self.steps_kv[st]
        bd.attn_packed(self.steps_q[st], pk, pv, self.k_eff, self.k_max, wk, wv, self.bl,
                       self.sm_scale, out=self.out, ws=self.ws_attn)

    def run_sequential(self, n_blocks: int):
        for n in range(n_blocks):
            self.retrieve(n % 2)
            for st in range(self.T):
                self.denoise(n % 2, st)
        return self.out

    def run_overlapped(self, n_blocks: int):
        main, ret = torch.cuda.current_stream(self.dev), self.retrieval
        ret.wait_stream(main)
        with torch.cuda.stream(ret):
            self.retrieve(0)
            self.ev_ready[0].record(ret)
        start_next = min(1, self.T - 1)   # after block n's second step
        for n in range(n_blocks):
            slot = n % 2
            main.wait_event(self.ev_ready[slot])
            for st in range(self.T):
                self.denoise(slot, st)
                if st == start_next and n + 1 < n_blocks:
                    self.ev_draft.record(main)
                    ret.wait_event(self.ev_draft)
                    with torch.cuda.stream(ret):
                        self.retrieve((n + 1) % 2)
                        self.ev_ready[(n + 1) % 2].record(ret)
        main.wait_stream(ret)
        return self.out
