/*
 * libbdattn: block-diffusion attention over a KV cache on AMD Instinct
 * MI355X (gfx950).
 *
 * Four operations make up the data-parallel hot path of block-diffusion
 * decoding with a KV cache:
 *
 *   bd_select       representative-query scan of the K cache plus a
 *                   per-KV-head top-k critical set
 *                   (HERALD, Sec. IV-A2 and Sec. IV-B4).
 *   bd_gather       copy of the selected entries into a compact pool
 *                   (HERALD, Sec. IV-B3; pools of Sec. IV-B1).
 *   bd_attn_packed  GQA attention of a packed window of W blocks over a
 *                   prefix (the cache, or a pool) plus the window, under the
 *                   per-row W-shaped mask with absolute offsets
 *                   (FlowBlock review, Eq. (5)-(6) = paper Eq. 4-5).
 *   bd_kv_scatter   write-back of the window's KV to its absolute positions
 *                   (FlowBlock review, Eq. (7) = paper Eq. 6).
 *
 * bd_qkv_rope_write produces the window's queries, keys and values from its
 * hidden states (projection + RoPE + cache write in one kernel).
 *
 * bd_attn_packed_dual runs bd_attn_packed for two row lists with different
 * prefix sources (cache rows and pool rows) in one launch.  bd_select_multi
 * is the exact selection in which every block query ranks the prefix (the
 * step HERALD reduces to one representative query).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Memory: every tensor pointer is device memory owned by the caller.  The
 *   library allocates nothing and keeps no state between calls; scratch
 *   space comes from a caller workspace whose size the matching
 *   *_workspace_size function returns (bd_attn_packed_noalloc instead uses
 *   one device array the library holds per GPU).
 * - Streams: every call is asynchronous on the given hipStream_t (passed as
 *   void*; NULL is the default stream).  No call synchronises, reads device
 *   memory from the host, or allocates, so calls can be captured in a HIP
 *   graph.  Host integers (s_max, k_max, p_max, ...) size the grids; the
 *   per-row values live in device int32 arrays.
 * - Layout: tensors are token-major with the head dimension d contiguous.
 *   Strides are in elements (int64) for the outer dimensions, e.g. a K cache
 *   [B, C, Hkv, d] has strides {C*Hkv*d, Hkv*d, d}.  Base pointers must be
 *   16-byte aligned and every stride times the element size a multiple of
 *   16 bytes.
 * - dtypes: BD_BF16 (bfloat16 storage, fp32 arithmetic) and BD_F32.
 * - Errors: host-side validation runs before any HIP call; on failure the
 *   call returns a nonzero bd_status, launches nothing and writes nothing.
 *   bd_last_error() returns a thread-local message for the last failure.
 * - Device-side values (offsets, lengths, indices) are range-checked in the
 *   kernels: an out-of-range value never causes an out-of-bounds access;
 *   the affected row, slot or entry is skipped (left unchanged) or clamped,
 *   as each function states.
 * - GQA: query head hq reads KV head hq / (Hq / Hkv).
 */
#ifndef BDATTN_H
#define BDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BD_OK = 0,
  BD_ERR_INVALID_ARG = 1, /* bad size, pointer, stride or alignment      */
  BD_ERR_UNSUPPORTED = 2, /* valid but not built: dtype / head-dim combo */
  BD_ERR_HIP = 3,         /* a HIP launch reported an error              */
  BD_ERR_WORKSPACE = 4    /* workspace missing or too small              */
} bd_status;

typedef enum { BD_BF16 = 0, BD_F32 = 1 } bd_dtype;

typedef enum {
  BD_REP_MEAN = 0, /* mean of the nq given queries                       */
  BD_REP_ROW = 1   /* one query row (HERALD's block-centre [MASK] query) */
} bd_rep_mode;

/* Window part of the attention mask.  The window holds q / bl blocks
 * (groups) of bl queries and their keys; prefix keys are always visible.
 * Query i (group floor(i/bl)) sees window key w (group floor(w/bl)) when
 *   BD_MASK_BLOCK_CAUSAL  group(w) <= group(i)      FlowBlock review Eq. (6)
 *   BD_MASK_ISOLATED      group(w) == group(i)      HERALD Sec. IV-B2: the
 *                         denoising and draft groups of one forward see the
 *                         prefix but not each other
 *   BD_MASK_SHARED_FIRST  group(w) == group(i) or group(w) == 0
 *                         Flash-dLLM's verify pass: block 0 holds the
 *                         tracked context, later blocks are views that see
 *                         it but not each other, and it sees none of them */
typedef enum {
  BD_MASK_BLOCK_CAUSAL = 0,
  BD_MASK_ISOLATED = 1,
  BD_MASK_SHARED_FIRST = 2
} bd_mask_mode;

/* Library version string, e.g. "libbdattn 0.1.0 gfx950". */
const char *bd_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char *bd_last_error(void);

/*
 * bd_kv_scatter: FlowBlock review Eq. (7) (paper Eq. 6).
 *
 *   data[l, b, o_b + delta, h, :] <- present[l, b, t + delta, h, :]
 *   for delta < q, every KV head h and every layer l < n_layers,
 *
 * for the rows b listed in row_ids (all B rows when row_ids is NULL; then
 * n_rows must equal B).  Keys and values are both moved (data_v may be NULL
 * together with present_v to move K only).  Bit-exact copy of any dtype.
 *
 *   present_k/v  [n_layers, B, present_cap, Hkv, d], strides present_strides
 *                {layer, row, pos, head}; positions [t, t+q) are read.
 *   data_k/v     [n_layers, B, data_cap, Hkv, d], strides data_strides.
 *   o            device int32 [B]: per-row write offset o_b.
 *
 * present may alias data (the FlowBlock cache: window at the tail
 * t = C - q).  Requires t + q <= present_cap.  A row whose o_b is negative
 * or has o_b + q > data_cap is skipped; with aliasing, o_b must satisfy
 * o_b + q <= t or o_b == t, otherwise the result is undefined.
 */
int bd_kv_scatter(int dtype, int B, int Hkv, int d, int q, int n_layers,
                  const void *present_k, const void *present_v,
                  const int64_t present_strides[4], int present_cap, int t,
                  void *data_k, void *data_v, const int64_t data_strides[4],
                  int data_cap, const int32_t *o, const int32_t *row_ids,
                  int n_rows, void *stream);

/*
 * bd_gather: HERALD Sec. IV-B3 (CPU gather of the selected entries into a
 * contiguous buffer), here device memory to device memory.
 *
 *   k_pool[b, j, h, :] = k_src[b, idx[b, h, j], h, :]   for j < k_cnt[b]
 *   v_pool[b, j, h, :] = v_src[b, idx[b, h, j], h, :]
 *
 *   k_src/v_src  [B, src_cap, Hkv, d], strides src_strides {row, pos, head}.
 *   idx          device int32 [B, Hkv, k_max], contiguous (bd_select output).
 *   k_cnt        device int32 [B]; clamped to [0, k_max].
 *   k_pool/v_pool [B, pool_cap, Hkv, d], strides pool_strides; pool_cap >= k_max.
 *
 * Pool slots j >= k_cnt[b] are left unchanged, as is any slot whose index is
 * outside [0, src_cap).  v_src/v_pool may both be NULL to gather K only.
 */
int bd_gather(int dtype, int B, int Hkv, int d, const void *k_src,
              const void *v_src, const int64_t src_strides[3], int src_cap,
              const int32_t *idx, int k_max, const int32_t *k_cnt,
              void *k_pool, void *v_pool, const int64_t pool_strides[3],
              int pool_cap, void *stream);

/*
 * bd_select: HERALD Sec. IV-A2 (representative query) and Sec. IV-B4
 * (fused selection: GQA importance and one top-k per KV head).
 *
 * For every row b with S_b = s_len[b] > 0 and k_b = k_sel[b] > 0:
 *   q_rep[hq]   = mean_i q[b, i, hq, :] over i < nq     (BD_REP_MEAN)
 *               = q[b, rep_row, hq, :]                  (BD_REP_ROW)
 *   z[g, s]     = sm_scale * <q_rep[h*G+g], k[b, s, h, :]>   for s < S_b
 *   m_g, l_g    = max_s z[g, s],  sum_s exp(z[g, s] - m_g)
 *   score[h, s] = sum_g exp(z[g, s] - m_g) / l_g
 *   idx_out[b, h, 0:min(k_b, S_b)] = the positions of the min(k_b, S_b)
 *       largest scores, ties to the lower position, in ascending order;
 *       the remaining slots up to k_max hold -1.
 * Rows with S_b == 0 or k_b == 0 get idx_out all -1.
 *
 *   q         [B, nq, Hq, d] bf16, strides q_strides {row, query, head}.
 *   k         [B, k_cap, Hkv, d] bf16, strides k_strides.
 *   s_len     device int32 [B], clamped to [0, min(s_max, k_cap)].
 *   k_sel     device int32 [B], clamped to [0, k_max].
 *   idx_out   device int32 [B, Hkv, k_max], contiguous.
 *   score_out optional device float [B, Hkv, s_max], contiguous: receives
 *             the score vector exactly as ranked (positions >= S_b, and rows
 *             with S_b == 0 or k_b == 0, are not written).  NULL keeps the
 *             scores in the workspace.
 *   workspace at least bd_select_workspace_size(...) bytes, 256-byte aligned.
 *
 * Built for dtype BD_BF16 with d == 128 and Hq / Hkv <= 8.
 */
size_t bd_select_workspace_size(int B, int Hq, int Hkv, int d, int s_max,
                                int k_max);
int bd_select(int dtype, int B, int Hq, int Hkv, int d, const void *q,
              const int64_t q_strides[3], int nq, int rep_mode, int rep_row,
              const void *k, const int64_t k_strides[3], int k_cap,
              const int32_t *s_len, int s_max, const int32_t *k_sel, int k_max,
              float sm_scale, int32_t *idx_out, float *score_out,
              void *workspace, size_t ws_bytes, void *stream);

/*
 * bd_select_attn: bd_select plus the representative query's attention
 * output, HERALD Sec. IV-B4: beside the importance scores the fused
 * selection kernel keeps, for every query head g, the FlashAttention running
 * statistics (m_g, l_g) and output o_g, and the attention output goes back at
 * once so that the layer's FFN can run.
 *
 * Everything bd_select computes, with the same arguments and results, plus,
 * for every row b with S_b > 0 and k_b > 0 and query head hq = h*G + g:
 *   o_rep[b, hq, :] = sum_{s < S_b} exp(z[g, s] - m_g) / l_g * v[b, s, h, :]
 * (softmax attention of q_rep over the row's prefix; z, m_g, l_g as in
 * bd_select, the same weights whose sums over g are the ranked scores).
 * Rows with S_b == 0 or k_b == 0 get o_rep all zeros.
 *
 *   v         [B, k_cap, Hkv, d] bf16, strides v_strides {row, position,
 *             head}, 16-byte aligned with 16-byte stride multiples.
 *   o_rep     device bf16 [B, Hq, d], contiguous; required.
 *   idx_out   may be NULL when k_max == 0 (o_rep is then all zeros).
 *   workspace at least bd_select_attn_workspace_size(...) bytes, 256-byte
 *             aligned (bd_select's plus fp32 output partials per 1024
 *             prefix positions).
 *
 * Built for dtype BD_BF16 with d == 128 and Hq / Hkv <= 8.
 */
size_t bd_select_attn_workspace_size(int B, int Hq, int Hkv, int d, int s_max,
                                     int k_max);
int bd_select_attn(int dtype, int B, int Hq, int Hkv, int d, const void *q,
                   const int64_t q_strides[3], int nq, int rep_mode,
                   int rep_row, const void *k, const int64_t k_strides[3],
                   const void *v, const int64_t v_strides[3], int k_cap,
                   const int32_t *s_len, int s_max, const int32_t *k_sel,
                   int k_max, float sm_scale, int32_t *idx_out,
                   float *score_out, void *o_rep, void *workspace,
                   size_t ws_bytes, void *stream);

/*
 * bd_select_multi: exact multi-query selection, the selection phase of
 * HERALD Sec. III-C / Sec. IV-A2 before the query reduction (every block
 * query ranks the prefix, as in MAGE's full-KV selection at a block's first
 * step; Fig. 8 sweeps the number of queries).
 *
 * For every row b with S_b = s_len[b] > 0 and k_b = k_sel[b] > 0, KV head h,
 * query i < nq and group head g < G = Hq / Hkv:
 *   z[i, g, s]  = sm_scale * <q[b, i, h*G+g], k[b, s, h, :]>   for s < S_b
 *   m_ig, l_ig  = max_s z[i, g, s],  sum_s exp(z[i, g, s] - m_ig)
 *   score[h, s] = sum_i sum_g exp(z[i, g, s] - m_ig) / l_ig
 * (the per-query probabilities are summed like the group heads' in
 * Sec. IV-B4; nq = 1 gives bd_select's score with that query), and idx_out
 * as in bd_select: the positions of the min(k_b, S_b) largest scores, ties to
 * the lower position, ascending, -1 padded to k_max.
 *
 * Arguments, layouts, clamping and score_out are those of bd_select; q holds
 * the nq raw block queries [B, nq, Hq, d] (no mean is taken).  The logits are
 * bf16 products accumulated in fp32; K is read twice (statistics, then
 * scores), the score matrix is never stored.
 *   workspace at least bd_select_multi_workspace_size(...) bytes, 256-byte
 *             aligned.
 *
 * Built for dtype BD_BF16 with d == 128 and nq * Hq / Hkv <= 128.
 */
size_t bd_select_multi_workspace_size(int B, int Hq, int Hkv, int d, int nq,
                                      int s_max, int k_max);
int bd_select_multi(int dtype, int B, int Hq, int Hkv, int d, const void *q,
                    const int64_t q_strides[3], int nq, const void *k,
                    const int64_t k_strides[3], int k_cap,
                    const int32_t *s_len, int s_max, const int32_t *k_sel,
                    int k_max, float sm_scale, int32_t *idx_out,
                    float *score_out, void *workspace, size_t ws_bytes,
                    void *stream);

/*
 * bd_attn_packed: FlowBlock review Eq. (6) (paper Eq. 5) in prefix/window
 * form; HERALD's denoising attention when the prefix is a pool.
 *
 * For each listed row b, query i < q, query head hq (KV head h):
 *   visible keys = prefix entries pk/pv[b, j, h] for j < P_b = p_len[b]
 *                  and window entries wk/wv[b, w, h] for
 *                  w < (floor(i / bl) + 1) * bl      (capped at q)
 *   out[b, i, hq, :] = sum_j softmax_j(sm_scale * <q[b,i,hq], key_j>) value_j
 *   lse[b, hq, i]    = log sum_j exp(sm_scale * <q[b,i,hq], key_j>)
 *
 * FlowBlock call: pk = the cache [B, C, Hkv, d], p_len = o, wk = cache + t *
 * pos_stride with t = C - q: key j < o_b is prefix j and key j in [t, C) is
 * window j - t, exactly the Eq. (6) mask.  Sparse call: pk = a pool filled
 * by bd_gather, p_len = k_b.  q = W * bl for a window of W blocks.
 *
 *   row_ids   device int32 [n_rows] or NULL (all B rows; n_rows == B).
 *             Rows not listed are not written.  Entries outside [0, B) are
 *             skipped.
 *   q, out    [B, q, Hq, d], strides {row, query, head}.  out has q's dtype.
 *   pk/pv     [B, p_cap, Hkv, d]; p_len device int32 [B], clamped to
 *             [0, min(p_max, p_cap)].  Prefix rows at or past P_b are never
 *             read, so they may hold anything (NaN included).  Every visible
 *             key and value, and every query, must be finite: the kernels
 *             are built without NaN semantics (maxima take no NaN-quieting
 *             step), so a NaN or infinity there gives an unspecified
 *             output, not necessarily NaN.
 *   wk/wv     [B, q, Hkv, d] (any strides, e.g. a view of the cache tail).
 *   lse       optional device float [B, Hq, q], contiguous.
 *   workspace at least bd_attn_workspace_size(...) bytes, 256-byte aligned
 *             (zero bytes are needed when the split plan keeps one chunk).
 *
 * Built for: BD_BF16 with d == 128 and Hq / Hkv in {1, 2, 4, 8} (MFMA path),
 * BD_BF16 / BD_F32 with d in {64, 128} (general path).
 */
size_t bd_attn_workspace_size(int dtype, int B, int Hq, int Hkv, int d, int q,
                              int n_rows, int p_max);
int bd_attn_packed(int dtype, int B, int Hq, int Hkv, int d, int q, int bl,
                   const int32_t *row_ids, int n_rows, const void *q_ptr,
                   const int64_t q_strides[3], const void *pk, const void *pv,
                   const int64_t p_strides[3], int p_cap,
                   const int32_t *p_len, int p_max, const void *wk,
                   const void *wv, const int64_t w_strides[3], float sm_scale,
                   void *out, const int64_t out_strides[3], float *lse,
                   void *workspace, size_t ws_bytes, void *stream);

/*
 * bd_attn_packed_masked: bd_attn_packed with the window mask chosen by
 * mask_mode (bd_mask_mode): BD_MASK_BLOCK_CAUSAL is bd_attn_packed;
 * BD_MASK_ISOLATED is HERALD's fused draft/denoise forward (Sec. IV-B2);
 * BD_MASK_SHARED_FIRST is Flash-dLLM's verify views.  Every query still sees
 * its whole prefix and its own block.  Other arguments, layouts and errors as
 * bd_attn_packed; an unknown mode returns BD_ERR_INVALID_ARG.
 */
int bd_attn_packed_masked(int dtype, int B, int Hq, int Hkv, int d, int q,
                          int bl, int mask_mode,
                          const int32_t *row_ids, int n_rows, const void *q_ptr,
                          const int64_t q_strides[3], const void *pk, const void *pv,
                          const int64_t p_strides[3], int p_cap,
                          const int32_t *p_len, int p_max, const void *wk,
                          const void *wv, const int64_t w_strides[3], float sm_scale,
                          void *out, const int64_t out_strides[3], float *lse,
                          void *workspace, size_t ws_bytes, void *stream);

/*
 * bd_attn_packed_dual: bd_attn_packed over two row lists in one launch,
 * each list with its own prefix source.  The rows of list a attend over
 * pk_a/pv_a with lengths p_len_a, the rows of list b over pk_b/pv_b with
 * lengths p_len_b; the queries, the window source and the output are
 * shared.  The mask and the result of every row are exactly those of
 * bd_attn_packed with that row's source (FlowBlock review Eq. (6) when the
 * source is the cache; HERALD's denoising attention, Sec. III-C and
 * Sec. IV-B1, when it is a pool).  It serves a batch whose rows are split
 * between dense attention over their own cache and sparse attention over a
 * gathered pool: one launch lets the short pool rows fill the tail of the
 * long cache rows.
 *
 *   rows_a, rows_b  device int32 [n_a], [n_b]; required when the count is
 *                   positive.  Entries outside [0, B) are skipped; a row in
 *                   both lists is written by both (the result is one of
 *                   the two).
 *   pk_x/pv_x       [B, pX_cap, Hkv, d] with strides pX_strides; p_len_x
 *                   device int32 [B], clamped to [0, min(p_max_x, pX_cap)].
 *   everything else as in bd_attn_packed; the workspace is at least
 *   bd_attn_dual_workspace_size(...) bytes.
 *
 * Errors as bd_attn_packed.  Built for the same dtype / d / GQA shapes.
 */
size_t bd_attn_dual_workspace_size(int dtype, int B, int Hq, int Hkv, int d,
                                   int q, int n_a, int p_max_a, int n_b,
                                   int p_max_b);
int bd_attn_packed_dual(int dtype, int B, int Hq, int Hkv, int d, int q,
                        int bl, const void *q_ptr, const int64_t q_strides[3],
                        const int32_t *rows_a, int n_a, const void *pk_a,
                        const void *pv_a, const int64_t pa_strides[3],
                        int pa_cap, const int32_t *p_len_a, int p_max_a,
                        const int32_t *rows_b, int n_b, const void *pk_b,
                        const void *pv_b, const int64_t pb_strides[3],
                        int pb_cap, const int32_t *p_len_b, int p_max_b,
                        const void *wk, const void *wv,
                        const int64_t w_strides[3], float sm_scale, void *out,
                        const int64_t out_strides[3], float *lse,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * bd_attn_packed_noalloc: bd_attn_packed for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, mask, results and errors
 * as bd_attn_packed, minus the workspace: the call's scratch (row order and
 * split-prefix partials, bd_attn_workspace_size(...) bytes) lives in a
 * device array of BD_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends.  The call allocates nothing and
 * calls no allocating routine; a call whose scratch would exceed
 * BD_NOALLOC_SCRATCH_BYTES returns BD_ERR_WORKSPACE before any HIP call.
 * Every call on one GPU shares that array: calls that overlap on one GPU
 * (on two streams) race and must not be issued.  The first call on a device
 * looks up the array's address there (a non-allocating runtime query).
 */
#define BD_NOALLOC_SCRATCH_BYTES (32u << 20)
int bd_attn_packed_noalloc(int dtype, int B, int Hq, int Hkv, int d, int q, int bl,
                           const int32_t *row_ids, int n_rows, const void *q_ptr,
                           const int64_t q_strides[3], const void *pk, const void *pv,
                           const int64_t p_strides[3], int p_cap, const int32_t *p_len,
                           int p_max, const void *wk, const void *wv,
                           const int64_t w_strides[3], float sm_scale, void *out,
                           const int64_t out_strides[3], float *lse, void *stream);

/*
 * bd_attn_block_table: Flash-dLLM's Scheduled Flash Attention (Flash-Cache,
 * Fig. 3(b)): the batch is cut into work items, and a block table aligns
 * each item's query block with the key-value blocks it attends over; the
 * caller controls which blocks are computed and in what order, and adds or
 * removes items freely between calls.  Here the key-value blocks are pages
 * of a paged KV store (any page anywhere, in any order), and every item
 * also attends over its row's window under the FlowBlock mask, so a
 * contiguous table gives exactly bd_attn_packed (FlowBlock review Eq. (6);
 * HERALD's denoising attention when the pages hold a gathered pool).
 *
 * For each item e = items[n] (n < n_items) with row b = e.row, query
 * i in [e.q_begin, min(e.q_end, q)) and query head hq (KV head h):
 *   visible keys = the first L = min(e.kv_len, kv_max) keys of the pages
 *                  table[e.table_off + j], j < ceil(L / page), in that order
 *                  (key m of the list is position m % page of page
 *                  table[e.table_off + m / page]), and the window entries
 *                  wk/wv[b, w, h] with w < (floor(i / bl) + 1) * bl
 *   out[b, i, hq, :], lse[b, hq, i] as in bd_attn_packed.
 *
 *   items     device bd_attn_item [n_items], dispatched in list order.
 *             An item whose row is outside [0, B), whose query range is
 *             empty, or whose pages run past n_table is skipped.  Items
 *             must cover disjoint (row, query) sets: outputs no item covers
 *             are not written; two items covering the same output leave one
 *             of the two results.
 *   table     device int32 [n_table]: page ids; a page id outside
 *             [0, n_pages) contributes no keys.
 *   kv_k/kv_v the paged store [n_pages, page, Hkv, d], strides kv_strides
 *             {page, pos, head}; page a multiple of 64 keys (one 64-key
 *             tile never straddles two pages).
 *   q, wk/wv, out, lse, sm_scale as in bd_attn_packed.
 *   workspace at least bd_attn_block_table_workspace_size(...) bytes,
 *             256-byte aligned (split partials when few items).
 *
 * Built for BD_BF16 with d == 128 and Hq / Hkv in {1, 2, 4, 8}; other
 * combinations return BD_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t row;       /* row b of q, the window and out                     */
  int32_t q_begin;   /* first window query of the item                     */
  int32_t q_end;     /* one past its last window query (clamped to q)      */
  int32_t table_off; /* first entry of the item's pages in the table       */
  int32_t kv_len;    /* keys on those pages (clamped to [0, kv_max])       */
} bd_attn_item;

size_t bd_attn_block_table_workspace_size(int dtype, int Hq, int Hkv, int d, int q,
                                          int n_items, int kv_max);
int bd_attn_block_table(int dtype, int B, int Hq, int Hkv, int d, int q, int bl,
                        const bd_attn_item *items, int n_items,
                        const int32_t *table, int n_table, const void *kv_k,
                        const void *kv_v, const int64_t kv_strides[3],
                        int n_pages, int page, int kv_max, const void *q_ptr,
                        const int64_t q_strides[3], const void *wk,
                        const void *wv, const int64_t w_strides[3],
                        float sm_scale, void *out,
                        const int64_t out_strides[3], float *lse,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * bd_qkv_rope_write: Flash-dLLM's fused cache producer (Flash-Cache): the
 * projection of the window's hidden states onto the query, key and value
 * heads, the rotary embedding of queries and keys at absolute positions
 * (HERALD Eq. (1); FlowBlock's packed windows use absolute-position RoPE),
 * and the write of keys and values into the cache, with no intermediate
 * tensor in memory.
 *
 * For row b < B, window token i < q (absolute position
 * p = rope_pos[b] + i) and head n < Hq + 2*Hkv (the Hq query heads, then the
 * Hkv key heads, then the Hkv value heads):
 *   y[n, :] = sum_e x[b, i, e] * w[n*d + :, e]          (fp32 accumulation)
 *   query and key heads: y[j], y[j + d/2] (j < d/2) rotate by the angle
 *   p * rope_base^(-2j/d):  y'[j] = y[j] cos - y[j+d/2] sin,
 *                           y'[j+d/2] = y[j+d/2] cos + y[j] sin
 *   q_out[b, i, n]                 = y'  (query heads)
 *   k_cache[b, dst_pos[b] + i, n-Hq] = y'  (key heads)
 *   v_cache[b, dst_pos[b] + i, n-Hq-Hkv] = y  (value heads)
 * all rounded once to bf16.  dst_pos[b] = C - q writes the window tail that
 * bd_attn_packed reads; dst_pos[b] = o_b writes straight to the Eq. (7)
 * position.  Cache positions outside [0, c_cap) are not written.
 *
 *   x         [B, q, Dm] bf16, strides x_strides {row, token}; Dm contiguous.
 *   w         [(Hq + 2*Hkv) * d, Dm] bf16, contiguous (a linear layer's weight).
 *   rope_pos, dst_pos  device int32 [B].
 *   q_out     [B, q, Hq, d] bf16, strides q_strides.
 *   k_cache, v_cache   [B, c_cap, Hkv, d] bf16, shared strides c_strides.
 *
 * Built for dtype BD_BF16 with d == 128 and Dm a multiple of 64; W and the
 * span of x each under 2 GiB (BD_ERR_UNSUPPORTED otherwise).
 */
int bd_qkv_rope_write(int dtype, int B, int q, int Dm, int Hq, int Hkv, int d,
                      const void *x, const int64_t x_strides[2], const void *w,
                      const int32_t *rope_pos, float rope_base, void *q_out,
                      const int64_t q_strides[3], void *k_cache, void *v_cache,
                      const int64_t c_strides[3], int c_cap,
                      const int32_t *dst_pos, void *stream);

/*
 * Device check mode.  The per-row values the operations read from device
 * memory (row ids, lengths, offsets, gather indices, page tables) are
 * range-checked in the kernels, which clamp or skip what is out of range
 * without any out-of-bounds access, silently.  A caller that wants to know
 * calls the matching bd_check_* function on the same stream before the
 * operation, with the same values: it ORs one BD_CHECK_* bit per kind of
 * violation into *status (a device uint32 the caller clears; the checks
 * never clear it, so several can share one word) and writes nothing else.
 * The checks are asynchronous, allocate nothing and can be captured in a HIP
 * graph.  (No page states a status word: this is the caller's view of the
 * contract of each operation, as its comment above states it.)
 *
 * Host-side argument errors are returned as for the operations
 * (BD_ERR_INVALID_ARG with bd_last_error(); nothing is launched).
 */
#define BD_CHECK_ROW     0x01u /* a row id outside [0, B)                     */
#define BD_CHECK_LENGTH  0x02u /* a per-row length outside its range (p_len,
                                  s_len, k_sel, k_cnt, kv_len): clamped       */
#define BD_CHECK_OFFSET  0x04u /* a scatter offset with o_b < 0 or
                                  o_b + q > data_cap: row skipped              */
#define BD_CHECK_ALIAS   0x08u /* an aliased scatter whose target overlaps its
                                  source window (o_b + q > t and o_b != t)     */
#define BD_CHECK_INDEX   0x10u /* a gather index outside [0, src_cap) in a
                                  row's first k_cnt slots: slot left unchanged */
#define BD_CHECK_PAGE    0x20u /* a page id outside [0, n_pages) (no keys), or
                                  an item's pages past the table (skipped)     */
#define BD_CHECK_QUERIES 0x40u /* an item's query range empty or starting
                                  outside [0, q): item skipped                 */

/* bd_attn_packed (and _masked, _noalloc; each list of _dual): row ids in
 * [0, B) (row_ids NULL = rows 0 .. n_rows-1) and p_len[b] in
 * [0, min(p_max, p_cap, p_hi)].  p_hi is the caller's own bound: t = C - q
 * for the FlowBlock call, where a prefix past t would overlap the window
 * tail; p_cap (or anything larger) otherwise. */
int bd_check_attn(int B, const int32_t *row_ids, int n_rows, const int32_t *p_len,
                  int p_max, int p_cap, int p_hi, uint32_t *status, void *stream);
/* bd_kv_scatter: row ids in [0, B); o_b >= 0 and o_b + q <= data_cap; with
 * aliased != 0 (present and data are one tensor) also o_b + q <= t or
 * o_b == t. */
int bd_check_scatter(int B, int q, int t, int data_cap, const int32_t *o,
                     const int32_t *row_ids, int n_rows, int aliased,
                     uint32_t *status, void *stream);
/* bd_gather: k_cnt[b] in [0, k_max] and idx[b, h, j] in [0, src_cap) for
 * j < k_cnt[b] (idx [B, Hkv, k_max], contiguous). */
int bd_check_gather(int B, int Hkv, const int32_t *idx, int k_max,
                    const int32_t *k_cnt, int src_cap, uint32_t *status,
                    void *stream);
/* bd_select / bd_select_multi: s_len[b] in [0, min(s_max, k_cap)] and
 * k_sel[b] in [0, k_max]. */
int bd_check_select(int B, const int32_t *s_len, int s_max, int k_cap,
                    const int32_t *k_sel, int k_max, uint32_t *status,
                    void *stream);
/* bd_attn_block_table: every item's row in [0, B), q_begin in [0, q) with
 * q_end > q_begin, kv_len in [0, kv_max], table_off >= 0 with its
 * ceil(kv_len / page) pages inside the table, and every one of those page
 * ids in [0, n_pages). */
int bd_check_block_table(int B, int q, const bd_attn_item *items, int n_items,
                         const int32_t *table, int n_table, int n_pages,
                         int page, int kv_max, uint32_t *status, void *stream);

/*
 * bd_mask_materialize: test hook for the attention mask.  Writes
 * out[b, i, j] = 1 if query i of row b sees cache position j under
 * FlowBlock review Eq. (6) (j < o_b, or t <= j < t + (floor(i/bl)+1)*bl
 * with t = C - q; with another bd_mask_mode the tail part follows that
 * mode), else 0, for j < C.  out is device uint8 [B, q, C], contiguous.  It
 * evaluates the same device predicate the attention kernels use.  Rows with
 * o_b outside [0, t] are written all 0xFF.  Unknown modes return
 * BD_ERR_INVALID_ARG.
 */
int bd_mask_materialize(int B, int C, int q, int bl, int mask_mode,
                        const int32_t *o, uint8_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BDATTN_H */
