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
            bd.gather(self.Kc, self.Vc, self.idx, self.k_sel, self.pool_k, self.pool_v)

    def attn_dense(self):
        if self.n_dense:
            bd.attn_packed(self.Q, self.Kc, self.Vc, self.o, self.p_max_dense, self.wk, self.wv,
                           self.bl, self.sm_scale, out=self.out, row_ids=self.dense_rows,
                           ws=self.ws_dense)

    def attn_sparse(self):
        if self.n_sparse:
            bd.attn_packed(self.Q, self.pool_k, self.pool_v, self.k_sel, self.k_max, self.wk,
                           self.wv, self.bl, self.sm_scale, out=self.out,
                           row_ids=self.sparse_rows, ws=self.ws_sparse)

    def attn(self):
        """Attention of every row in one launch."""
        if self.n_dense and self.n_sparse:
            bd.attn_packed_dual(self.Q, (self.dense_rows, self.Kc, self.Vc, self.o, self.p_max_dense),
                                (self.sparse_rows, self.pool_k, self.pool_v, self.k_sel, self.k_max),
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
