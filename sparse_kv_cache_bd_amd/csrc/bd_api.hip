// Public C-ABI of libbdattn: argument validation (before any HIP call) and
// dispatch to the kernel launchers.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <stdint.h>

#include "bd_common.h"

namespace bd {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

static int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

static int esize(int dtype) { return dtype == BD_BF16 ? 2 : (dtype == BD_F32 ? 4 : 0); }

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static bool strides_ok(const int64_t *s, int n, int es) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || ((s[i] * es) & 15) != 0) return false;
  return true;
}

static int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return BD_OK;
  return fail(BD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace bd

using namespace bd;

extern "C" {

const char *bd_version(void) { return "libbdattn 0.1.0 gfx950"; }

const char *bd_last_error(void) { return g_err; }

int bd_kv_scatter(int dtype, int B, int Hkv, int d, int q, int n_layers, const void *present_k,
                  const void *present_v, const int64_t present_strides[4], int present_cap, int t,
                  void *data_k, void *data_v, const int64_t data_strides[4], int data_cap,
                  const int32_t *o, const int32_t *row_ids, int n_rows, void *stream) {
  g_err[0] = 0;
  const int es = esize(dtype);
  if (!es) return fail(BD_ERR_UNSUPPORTED, "bd_kv_scatter: unknown dtype %d", dtype);
  if (B < 0 || Hkv <= 0 || d <= 0 || q < 0 || n_layers < 0 || n_rows < 0)
    return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: negative or zero size");
  if (!row_ids && n_rows != B)
    return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: n_rows must equal B when row_ids is NULL");
  if (B == 0 || q == 0 || n_layers == 0 || n_rows == 0) return BD_OK;
  if ((d * es) % 16 != 0)
    return fail(BD_ERR_UNSUPPORTED, "bd_kv_scatter: d * element size must be a multiple of 16 bytes");
  if ((int64_t)Hkv * d * es > 16384)
    return fail(BD_ERR_UNSUPPORTED, "bd_kv_scatter: one position of all KV heads exceeds 16 KB");
  if (!present_strides || !data_strides || !o)
    return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: null strides or offsets");
  if (!present_k || !data_k) return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: null K pointers");
  if ((present_v == nullptr) != (data_v == nullptr))
    return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: present_v and data_v must both be set or both NULL");
  if (t < 0 || (int64_t)t + q > present_cap)
    return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: window [t, t+q) = [%d, %d) outside present (cap %d)",
                t, t + q, present_cap);
  if (data_cap < q) return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: data_cap %d < q %d", data_cap, q);
  if (n_rows > 65535 || n_layers * 2 > 65535)
    return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: too many rows or layers for one launch");
  if (!strides_ok(present_strides, 4, es) || !strides_ok(data_strides, 4, es))
    return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: strides must be >= 0 and 16-byte multiples");
  if (!aligned16(present_k) || !aligned16(data_k) || (present_v && (!aligned16(present_v) || !aligned16(data_v))))
    return fail(BD_ERR_INVALID_ARG, "bd_kv_scatter: base pointers must be 16-byte aligned");
  ScatterArgs a;
  a.es = es; a.B = B; a.Hkv = Hkv; a.d = d; a.q = q; a.n_layers = n_layers; a.n_rows = n_rows;
  a.t = t; a.present_cap = present_cap; a.data_cap = data_cap;
  a.pk = (const char *)present_k; a.pv = (const char *)present_v;
  a.dk = (char *)data_k; a.dv = (char *)data_v;
  memcpy(a.ps, present_strides, sizeof(a.ps));
  memcpy(a.ds, data_strides, sizeof(a.ds));
  a.o = o; a.row_ids = row_ids;
  return hip_status(launch_scatter(a, (hipStream_t)stream), "bd_kv_scatter launch");
}

int bd_gather(int dtype, int B, int Hkv, int d, const void *k_src, const void *v_src,
              const int64_t src_strides[3], int src_cap, const int32_t *idx, int k_max,
              const int32_t *k_cnt, void *k_pool, void *v_pool, const int64_t pool_strides[3],
              int pool_cap, void *stream) {
  g_err[0] = 0;
  const int es = esize(dtype);
  if (!es) return fail(BD_ERR_UNSUPPORTED, "bd_gather: unknown dtype %d", dtype);
  if (B < 0 || Hkv <= 0 || d <= 0 || k_max < 0 || src_cap < 0)
    return fail(BD_ERR_INVALID_ARG, "bd_gather: negative or zero size");
  if (B == 0 || k_max == 0) return BD_OK;
  if ((d * es) % 16 != 0)
    return fail(BD_ERR_UNSUPPORTED, "bd_gather: d * element size must be a multiple of 16 bytes");
  if (d * es > 16384) return fail(BD_ERR_UNSUPPORTED, "bd_gather: one head row exceeds 16 KB");
  if (!k_src || !k_pool || !idx || !k_cnt || !src_strides || !pool_strides)
    return fail(BD_ERR_INVALID_ARG, "bd_gather: null pointer");
  if ((v_src == nullptr) != (v_pool == nullptr))
    return fail(BD_ERR_INVALID_ARG, "bd_gather: v_src and v_pool must both be set or both NULL");
  if (pool_cap < k_max) return fail(BD_ERR_INVALID_ARG, "bd_gather: pool_cap %d < k_max %d", pool_cap, k_max);
  if ((int64_t)B * Hkv > 65535) return fail(BD_ERR_INVALID_ARG, "bd_gather: B * Hkv too large");
  if (!strides_ok(src_strides, 3, es) || !strides_ok(pool_strides, 3, es))
    return fail(BD_ERR_INVALID_ARG, "bd_gather: strides must be >= 0 and 16-byte multiples");
  if (!aligned16(k_src) || !aligned16(k_pool) || (v_src && (!aligned16(v_src) || !aligned16(v_pool))))
    return fail(BD_ERR_INVALID_ARG, "bd_gather: base pointers must be 16-byte aligned");
  GatherArgs a;
  a.es = es; a.B = B; a.Hkv = Hkv; a.d = d; a.src_cap = src_cap; a.k_max = k_max; a.pool_cap = pool_cap;
  a.ks = (const char *)k_src; a.vs = (const char *)v_src;
  a.kp = (char *)k_pool; a.vp = (char *)v_pool;
  memcpy(a.ss, src_strides, sizeof(a.ss));
  memcpy(a.pls, pool_strides, sizeof(a.pls));
  a.idx = idx; a.k_cnt = k_cnt;
  return hip_status(launch_gather(a, (hipStream_t)stream), "bd_gather launch");
}

size_t bd_select_workspace_size(int B, int Hq, int Hkv, int d, int s_max, int k_max) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || s_max < 0 || k_max < 0) return 0;
  return select_workspace(B, Hq, Hkv, d, s_max, k_max);
}

// bd_select and bd_select_attn: the same checks and launch; v / v_strides /
// o_rep are null for bd_select.
static int select_impl(const char *fn, int dtype, int B, int Hq, int Hkv, int d, const void *q,
                       const int64_t q_strides[3], int nq, int rep_mode, int rep_row, const void *k,
                       const int64_t k_strides[3], const void *v, const int64_t v_strides[3], int k_cap,
                       const int32_t *s_len, int s_max, const int32_t *k_sel, int k_max, float sm_scale,
                       int32_t *idx_out, float *score_out, void *o_rep, void *workspace, size_t ws_bytes,
                       void *stream) {
  g_err[0] = 0;
  const bool with_out = o_rep != nullptr;
  if (dtype != BD_BF16) return fail(BD_ERR_UNSUPPORTED, "%s: only BD_BF16 is built", fn);
  if (d != 128) return fail(BD_ERR_UNSUPPORTED, "%s: only d == 128 is built", fn);
  if (B < 0 || Hq <= 0 || Hkv <= 0 || s_max < 0 || k_max < 0 || k_cap < 0)
    return fail(BD_ERR_INVALID_ARG, "%s: negative or zero size", fn);
  if (Hq % Hkv != 0) return fail(BD_ERR_INVALID_ARG, "%s: Hq %% Hkv != 0", fn);
  if (Hq / Hkv > 8 || Hq > 64) return fail(BD_ERR_UNSUPPORTED, "%s: needs Hq/Hkv <= 8 and Hq <= 64", fn);
  if (B == 0 || (k_max == 0 && !with_out)) return BD_OK;
  if ((k_max > 0 && !idx_out) || !s_len || !k_sel) return fail(BD_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (s_max > 0 && (!q || !k || !q_strides || !k_strides))
    return fail(BD_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (with_out && s_max > 0 && (!v || !v_strides)) return fail(BD_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (rep_mode != BD_REP_MEAN && rep_mode != BD_REP_ROW)
    return fail(BD_ERR_INVALID_ARG, "%s: unknown rep_mode %d", fn, rep_mode);
  if (nq <= 0) return fail(BD_ERR_INVALID_ARG, "%s: nq must be positive", fn);
  if (rep_mode == BD_REP_ROW && (rep_row < 0 || rep_row >= nq))
    return fail(BD_ERR_INVALID_ARG, "%s: rep_row %d outside [0, %d)", fn, rep_row, nq);
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return fail(BD_ERR_INVALID_ARG, "%s: bad sm_scale", fn);
  if ((int64_t)B * Hkv > 65535 || (int64_t)B * Hq > 65535 || B > 65535)
    return fail(BD_ERR_INVALID_ARG, "%s: too many rows for one launch", fn);
  if (s_max > 0 && (!strides_ok(q_strides, 3, 2) || !strides_ok(k_strides, 3, 2) || !aligned16(q) || !aligned16(k)))
    return fail(BD_ERR_INVALID_ARG, "%s: q/k must be 16-byte aligned with 16-byte stride multiples", fn);
  if (with_out && s_max > 0 && (!strides_ok(v_strides, 3, 2) || !aligned16(v)))
    return fail(BD_ERR_INVALID_ARG, "%s: v must be 16-byte aligned with 16-byte stride multiples", fn);
  const size_t need = select_workspace(B, Hq, Hkv, d, s_max, k_max, with_out);
  if (!workspace || ws_bytes < need)
    return fail(BD_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(BD_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  SelectArgs a;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.d = d; a.nq = nq; a.rep_mode = rep_mode;
  a.rep_row = rep_row; a.k_cap = k_cap; a.s_max = s_max; a.k_max = k_max;
  a.q = (const bf16 *)q; a.k = (const bf16 *)k;
  for (int i = 0; i < 3; ++i) { a.qs[i] = q_strides ? q_strides[i] : 0; a.ks[i] = k_strides ? k_strides[i] : 0; }
  a.s_len = s_len; a.k_sel = k_sel; a.scale2 = sm_scale * kLog2e;
  a.idx_out = idx_out; a.score_out = score_out; a.ws = (char *)workspace;
  a.v = (const bf16 *)v;
  for (int i = 0; i < 3; ++i) a.vs[i] = v_strides ? v_strides[i] : 0;
  a.o_rep = (bf16 *)o_rep;
  char what[64];
  snprintf(what, sizeof(what), "%s launch", fn);
  return hip_status(launch_select(a, (hipStream_t)stream), what);
}

int bd_select(int dtype, int B, int Hq, int Hkv, int d, const void *q, const int64_t q_strides[3],
              int nq, int rep_mode, int rep_row, const void *k, const int64_t k_strides[3], int k_cap,
              const int32_t *s_len, int s_max, const int32_t *k_sel, int k_max, float sm_scale,
              int32_t *idx_out, float *score_out, void *workspace, size_t ws_bytes, void *stream) {
  return select_impl("bd_select", dtype, B, Hq, Hkv, d, q, q_strides, nq, rep_mode, rep_row, k, k_strides,
                     nullptr, nullptr, k_cap, s_len, s_max, k_sel, k_max, sm_scale, idx_out, score_out,
                     nullptr, workspace, ws_bytes, stream);
}

size_t bd_select_attn_workspace_size(int B, int Hq, int Hkv, int d, int s_max, int k_max) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || s_max < 0 || k_max < 0 || Hq % Hkv != 0) return 0;
  return select_workspace(B, Hq, Hkv, d, s_max, k_max, true);
}

int bd_select_attn(int dtype, int B, int Hq, int Hkv, int d, const void *q, const int64_t q_strides[3],
                   int nq, int rep_mode, int rep_row, const void *k, const int64_t k_strides[3],
                   const void *v, const int64_t v_strides[3], int k_cap, const int32_t *s_len, int s_max,
                   const int32_t *k_sel, int k_max, float sm_scale, int32_t *idx_out, float *score_out,
                   void *o_rep, void *workspace, size_t ws_bytes, void *stream) {
  if (B > 0 && !o_rep) {
    g_err[0] = 0;
    return fail(BD_ERR_INVALID_ARG, "bd_select_attn: null pointer (o_rep)");
  }
  return select_impl("bd_select_attn", dtype, B, Hq, Hkv, d, q, q_strides, nq, rep_mode, rep_row, k,
                     k_strides, v, v_strides, k_cap, s_len, s_max, k_sel, k_max, sm_scale, idx_out,
                     score_out, o_rep, workspace, ws_bytes, stream);
}

size_t bd_select_multi_workspace_size(int B, int Hq, int Hkv, int d, int nq, int s_max, int k_max) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || nq <= 0 || s_max < 0 || k_max < 0) return 0;
  return select_multi_workspace(B, Hkv, s_max);
}

int bd_select_multi(int dtype, int B, int Hq, int Hkv, int d, const void *q, const int64_t q_strides[3],
                    int nq, const void *k, const int64_t k_strides[3], int k_cap, const int32_t *s_len,
                    int s_max, const int32_t *k_sel, int k_max, float sm_scale, int32_t *idx_out,
                    float *score_out, void *workspace, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (dtype != BD_BF16) return fail(BD_ERR_UNSUPPORTED, "bd_select_multi: only BD_BF16 is built");
  if (d != 128) return fail(BD_ERR_UNSUPPORTED, "bd_select_multi: only d == 128 is built");
  if (B < 0 || Hq <= 0 || Hkv <= 0 || s_max < 0 || k_max < 0 || k_cap < 0)
    return fail(BD_ERR_INVALID_ARG, "bd_select_multi: negative or zero size");
  if (Hq % Hkv != 0) return fail(BD_ERR_INVALID_ARG, "bd_select_multi: Hq %% Hkv != 0");
  if (nq <= 0) return fail(BD_ERR_INVALID_ARG, "bd_select_multi: nq must be positive");
  if ((int64_t)nq * (Hq / Hkv) > 128)
    return fail(BD_ERR_UNSUPPORTED, "bd_select_multi: needs nq * Hq/Hkv <= 128 (got %d * %d)", nq, Hq / Hkv);
  if (B == 0 || k_max == 0) return BD_OK;
  if (!idx_out || !s_len || !k_sel) return fail(BD_ERR_INVALID_ARG, "bd_select_multi: null pointer");
  if (s_max > 0 && (!q || !k || !q_strides || !k_strides))
    return fail(BD_ERR_INVALID_ARG, "bd_select_multi: null pointer");
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return fail(BD_ERR_INVALID_ARG, "bd_select_multi: bad sm_scale");
  if ((int64_t)B * Hkv > 65535 || B > 65535 || Hkv > 65535)
    return fail(BD_ERR_INVALID_ARG, "bd_select_multi: too many rows for one launch");
  if (s_max > 0 && (!strides_ok(q_strides, 3, 2) || !strides_ok(k_strides, 3, 2) || !aligned16(q) || !aligned16(k)))
    return fail(BD_ERR_INVALID_ARG, "bd_select_multi: q/k must be 16-byte aligned with 16-byte stride multiples");
  const size_t need = select_multi_workspace(B, Hkv, s_max);
  if (!workspace || ws_bytes < need)
    return fail(BD_ERR_WORKSPACE, "bd_select_multi: workspace %zu bytes, need %zu", ws_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(BD_ERR_WORKSPACE, "bd_select_multi: workspace must be 256-byte aligned");
  SelectArgs a;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.d = d; a.nq = nq; a.rep_mode = BD_REP_MEAN;
  a.rep_row = 0; a.k_cap = k_cap; a.s_max = s_max; a.k_max = k_max;
  a.q = (const bf16 *)q; a.k = (const bf16 *)k;
  for (int i = 0; i < 3; ++i) { a.qs[i] = q_strides ? q_strides[i] : 0; a.ks[i] = k_strides ? k_strides[i] : 0; }
  a.s_len = s_len; a.k_sel = k_sel; a.scale2 = sm_scale * kLog2e;
  a.idx_out = idx_out; a.score_out = score_out; a.ws = (char *)workspace;
  return hip_status(launch_select_multi(a, (hipStream_t)stream), "bd_select_multi launch");
}

size_t bd_attn_workspace_size(int dtype, int B, int Hq, int Hkv, int d, int q, int n_rows, int p_max) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || q <= 0 || n_rows <= 0 || p_max < 0) return 0;
  return attn_plan(dtype, B, Hq, Hkv, d, q, n_rows, p_max).ws_bytes;
}

size_t bd_attn_dual_workspace_size(int dtype, int B, int Hq, int Hkv, int d, int q, int n_a,
                                   int p_max_a, int n_b, int p_max_b) {
  if (n_a < 0 || n_b < 0 || p_max_a < 0 || p_max_b < 0) return 0;
  return bd_attn_workspace_size(dtype, B, Hq, Hkv, d, q, n_a + n_b, p_max_a > p_max_b ? p_max_a : p_max_b);
}

}  // extern "C"

namespace bd {

// Shared body of bd_attn_packed (one source), bd_attn_packed_dual (two) and
// bd_attn_packed_noalloc: validation before any HIP call, then the argument
// block and the launch plan.  *launch is false when there is nothing to do.
int attn_setup(const char *fn, int dtype, int B, int Hq, int Hkv, int d, int q, int bl,
               int mask_mode, const void *q_ptr, const int64_t q_strides[3], const PrefixArg &pa,
               const PrefixArg *pb, const void *wk, const void *wv, const int64_t w_strides[3],
               float sm_scale, void *out, const int64_t out_strides[3], float *lse,
               AttnArgs &a, AttnPlan &plan, bool *launch) {
  g_err[0] = 0;
  *launch = false;
  const int es = esize(dtype);
  if (!es) return fail(BD_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || q < 0 || bl <= 0)
    return fail(BD_ERR_INVALID_ARG, "%s: negative or zero size", fn);
  for (const PrefixArg *p : {&pa, pb}) {
    if (p && (p->n < 0 || p->cap < 0 || p->p_max < 0))
      return fail(BD_ERR_INVALID_ARG, "%s: negative row count, capacity or p_max", fn);
  }
  if (Hq % Hkv != 0) return fail(BD_ERR_INVALID_ARG, "%s: Hq %% Hkv != 0", fn);
  if (mask_mode != BD_MASK_BLOCK_CAUSAL && mask_mode != BD_MASK_ISOLATED && mask_mode != BD_MASK_SHARED_FIRST)
    return fail(BD_ERR_INVALID_ARG, "%s: unknown mask mode %d", fn, mask_mode);
  if (!pb && !pa.rows && pa.n != B)
    return fail(BD_ERR_INVALID_ARG, "%s: n_rows must equal B when row_ids is NULL", fn);
  if (pb && ((pa.n > 0 && !pa.rows) || (pb->n > 0 && !pb->rows)))
    return fail(BD_ERR_INVALID_ARG, "%s: null row list", fn);
  const int G = Hq / Hkv;
  if (!attn_mfma_supported(dtype, d, G) && !attn_generic_supported(dtype, d))
    return fail(BD_ERR_UNSUPPORTED, "%s: dtype %d with d %d is not built", fn, dtype, d);
  const int n_rows = pa.n + (pb ? pb->n : 0);
  if ((int64_t)pa.n + (pb ? pb->n : 0) > INT32_MAX / 2)
    return fail(BD_ERR_INVALID_ARG, "%s: too many rows", fn);
  if (B == 0 || n_rows == 0 || q == 0) return BD_OK;
  if (!q_ptr || !wk || !wv || !out || !q_strides || !w_strides || !out_strides)
    return fail(BD_ERR_INVALID_ARG, "%s: null pointer", fn);
  for (const PrefixArg *p : {&pa, pb}) {
    if (!p || p->n == 0) continue;
    if (!p->p_len || !p->strides) return fail(BD_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (p->p_max > 0 && (!p->pk || !p->pv)) return fail(BD_ERR_INVALID_ARG, "%s: null prefix pointers", fn);
    if (!strides_ok(p->strides, 3, es))
      return fail(BD_ERR_INVALID_ARG, "%s: strides must be >= 0 and 16-byte multiples", fn);
    if (p->p_max > 0 && (!aligned16(p->pk) || !aligned16(p->pv)))
      return fail(BD_ERR_INVALID_ARG, "%s: base pointers must be 16-byte aligned", fn);
    if (p->strides[1] * es * 64 > INT32_MAX)
      return fail(BD_ERR_INVALID_ARG, "%s: key row strides above 32 MB are not supported", fn);
  }
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return fail(BD_ERR_INVALID_ARG, "%s: bad sm_scale", fn);
  if (!strides_ok(q_strides, 3, es) || !strides_ok(w_strides, 3, es) || !strides_ok(out_strides, 3, es))
    return fail(BD_ERR_INVALID_ARG, "%s: strides must be >= 0 and 16-byte multiples", fn);
  if (!aligned16(q_ptr) || !aligned16(wk) || !aligned16(wv) || !aligned16(out))
    return fail(BD_ERR_INVALID_ARG, "%s: base pointers must be 16-byte aligned", fn);
  if (w_strides[1] * es * 64 > INT32_MAX)
    return fail(BD_ERR_INVALID_ARG, "%s: key row strides above 32 MB are not supported", fn);
  a.dtype = dtype; a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.d = d; a.q = q; a.bl = bl;
  a.mask_mode = mask_mode;
  a.n_rows = n_rows;
  a.Q = q_ptr; a.wk = wk; a.wv = wv; a.out = out; a.lse = lse;
  memcpy(a.qs, q_strides, sizeof(a.qs));
  memcpy(a.ws, w_strides, sizeof(a.ws));
  memcpy(a.os, out_strides, sizeof(a.os));
  const bool use_a = pa.n > 0;
  a.n_rows1 = pa.n;
  a.row_ids = pa.rows; a.p_len = use_a ? pa.p_len : nullptr;
  a.pk = pa.pk; a.pv = pa.pv; a.p_cap = pa.cap; a.p_max = use_a ? pa.p_max : 0;
  for (int i = 0; i < 3; ++i) a.ps[i] = use_a ? pa.strides[i] : 0;
  const bool use_b = pb && pb->n > 0;
  a.row_ids2 = use_b ? pb->rows : nullptr; a.p_len2 = use_b ? pb->p_len : nullptr;
  a.pk2 = use_b ? pb->pk : nullptr; a.pv2 = use_b ? pb->pv : nullptr;
  a.p_cap2 = use_b ? pb->cap : 0; a.p_max2 = use_b ? pb->p_max : 0;
  for (int i = 0; i < 3; ++i) a.ps2[i] = use_b ? pb->strides[i] : 0;
  a.scale2 = sm_scale * kLog2e;
  const int p_max = a.p_max > a.p_max2 ? a.p_max : a.p_max2;
  plan = attn_plan(dtype, B, Hq, Hkv, d, q, n_rows, p_max);
  a.nw = plan.nw; a.nqt = plan.nqt; a.chunk = plan.chunk; a.n_split = plan.n_split;
  const int64_t grid_units = (8 + (int64_t)n_rows * Hkv) * a.nqt * a.n_split;
  if (grid_units > ((int64_t)1 << 31) - 1 || (int64_t)n_rows * Hq * a.nqt * a.n_split > ((int64_t)1 << 31) - 1)
    return fail(BD_ERR_INVALID_ARG, "%s: problem too large for one launch", fn);
  a.row_order = nullptr;
  a.part_o = nullptr;
  a.gpart_o = nullptr;
  a.part_ml = nullptr;
  a.items = nullptr;
  a.table = nullptr;
  a.n_table = 0;
  a.page = 0;
  *launch = true;
  return BD_OK;
}

// Points the plan's scratch parts (row order, split partials) into ws.
void attn_bind_workspace(AttnArgs &a, const AttnPlan &plan, char *ws) {
  a.row_order = plan.order ? (int *)(ws + plan.off_order) : nullptr;
  a.part_o = plan.n_split > 1 && plan.nw > 0 ? (bf16 *)(ws + plan.off_part_o) : nullptr;
  a.gpart_o = plan.n_split > 1 && plan.nw == 0 ? (float *)(ws + plan.off_part_o) : nullptr;
  a.part_ml = plan.n_split > 1 ? (float *)(ws + plan.off_part_ml) : nullptr;
}

int attn_launch_status(hipError_t e, const char *fn) { return hip_status(e, fn); }

}  // namespace bd

namespace {

int attn_entry(const char *fn, int dtype, int B, int Hq, int Hkv, int d, int q, int bl,
               int mask_mode, const void *q_ptr, const int64_t q_strides[3], const PrefixArg &pa,
               const PrefixArg *pb, const void *wk, const void *wv, const int64_t w_strides[3],
               float sm_scale, void *out, const int64_t out_strides[3], float *lse,
               void *workspace, size_t ws_bytes, void *stream) {
  AttnArgs a;
  AttnPlan plan;
  bool launch;
  const int st = attn_setup(fn, dtype, B, Hq, Hkv, d, q, bl, mask_mode, q_ptr, q_strides, pa, pb,
                            wk, wv, w_strides, sm_scale, out, out_strides, lse, a, plan, &launch);
  if (st != BD_OK || !launch) return st;
  if (plan.ws_bytes > 0) {
    if (!workspace || ws_bytes < plan.ws_bytes)
      return fail(BD_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, plan.ws_bytes);
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(BD_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    attn_bind_workspace(a, plan, (char *)workspace);
  }
  return hip_status(launch_attn(a, (hipStream_t)stream), fn);
}

}  // namespace

extern "C" {

int bd_attn_packed(int dtype, int B, int Hq, int Hkv, int d, int q, int bl, const int32_t *row_ids,
                   int n_rows, const void *q_ptr, const int64_t q_strides[3], const void *pk,
                   const void *pv, const int64_t p_strides[3], int p_cap, const int32_t *p_len,
                   int p_max, const void *wk, const void *wv, const int64_t w_strides[3],
                   float sm_scale, void *out, const int64_t out_strides[3], float *lse,
                   void *workspace, size_t ws_bytes, void *stream) {
  const PrefixArg pa{row_ids, n_rows, pk, pv, p_strides, p_cap, p_len, p_max};
  return attn_entry("bd_attn_packed", dtype, B, Hq, Hkv, d, q, bl, BD_MASK_BLOCK_CAUSAL, q_ptr,
                    q_strides, pa, nullptr, wk, wv, w_strides, sm_scale, out, out_strides, lse,
                    workspace, ws_bytes, stream);
}

int bd_attn_packed_masked(int dtype, int B, int Hq, int Hkv, int d, int q, int bl, int mask_mode,
                          const int32_t *row_ids, int n_rows, const void *q_ptr,
                          const int64_t q_strides[3], const void *pk, const void *pv,
                          const int64_t p_strides[3], int p_cap, const int32_t *p_len, int p_max,
                          const void *wk, const void *wv, const int64_t w_strides[3],
                          float sm_scale, void *out, const int64_t out_strides[3], float *lse,
                          void *workspace, size_t ws_bytes, void *stream) {
  const PrefixArg pa{row_ids, n_rows, pk, pv, p_strides, p_cap, p_len, p_max};
  return attn_entry("bd_attn_packed_masked", dtype, B, Hq, Hkv, d, q, bl, mask_mode, q_ptr,
                    q_strides, pa, nullptr, wk, wv, w_strides, sm_scale, out, out_strides, lse,
                    workspace, ws_bytes, stream);
}

int bd_attn_packed_dual(int dtype, int B, int Hq, int Hkv, int d, int q, int bl, const void *q_ptr,
                        const int64_t q_strides[3], const int32_t *rows_a, int n_a, const void *pk_a,
                        const void *pv_a, const int64_t pa_strides[3], int pa_cap,
                        const int32_t *p_len_a, int p_max_a, const int32_t *rows_b, int n_b,
                        const void *pk_b, const void *pv_b, const int64_t pb_strides[3], int pb_cap,
                        const int32_t *p_len_b, int p_max_b, const void *wk, const void *wv,
                        const int64_t w_strides[3], float sm_scale, void *out,
                        const int64_t out_strides[3], float *lse, void *workspace, size_t ws_bytes,
                        void *stream) {
  const PrefixArg pa{rows_a, n_a, pk_a, pv_a, pa_strides, pa_cap, p_len_a, p_max_a};
  const PrefixArg pb{rows_b, n_b, pk_b, pv_b, pb_strides, pb_cap, p_len_b, p_max_b};
  return attn_entry("bd_attn_packed_dual", dtype, B, Hq, Hkv, d, q, bl, BD_MASK_BLOCK_CAUSAL, q_ptr, q_strides, pa, &pb,
                    wk, wv, w_strides, sm_scale, out, out_strides, lse, workspace, ws_bytes, stream);
}

size_t bd_attn_block_table_workspace_size(int dtype, int Hq, int Hkv, int d, int q, int n_items,
                                          int kv_max) {
  if (Hq <= 0 || Hkv <= 0 || d <= 0 || q <= 0 || n_items <= 0 || kv_max < 0) return 0;
  return attn_plan(dtype, 1, Hq, Hkv, d, q, n_items, kv_max, true).ws_bytes;
}

int bd_attn_block_table(int dtype, int B, int Hq, int Hkv, int d, int q, int bl,
                        const bd_attn_item *items, int n_items, const int32_t *table, int n_table,
                        const void *kv_k, const void *kv_v, const int64_t kv_strides[3],
                        int n_pages, int page, int kv_max, const void *q_ptr,
                        const int64_t q_strides[3], const void *wk, const void *wv,
                        const int64_t w_strides[3], float sm_scale, void *out,
                        const int64_t out_strides[3], float *lse, void *workspace, size_t ws_bytes,
                        void *stream) {
  static const char *fn = "bd_attn_block_table";
  g_err[0] = 0;
  const int es = esize(dtype);
  if (!es) return fail(BD_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || q < 0 || bl <= 0 || n_items < 0 || n_table < 0 ||
      n_pages < 0 || kv_max < 0)
    return fail(BD_ERR_INVALID_ARG, "%s: negative or zero size", fn);
  if (Hq % Hkv != 0) return fail(BD_ERR_INVALID_ARG, "%s: Hq %% Hkv != 0", fn);
  if (!attn_mfma_supported(dtype, d, Hq / Hkv))
    return fail(BD_ERR_UNSUPPORTED, "%s: built for bf16, d = 128, Hq/Hkv in {1, 2, 4, 8}", fn);
  if (page <= 0 || page % 64 != 0)
    return fail(BD_ERR_INVALID_ARG, "%s: page %d must be a positive multiple of 64 keys", fn, page);
  if (n_items > INT32_MAX / 2) return fail(BD_ERR_INVALID_ARG, "%s: too many items", fn);
  if (B == 0 || n_items == 0 || q == 0) return BD_OK;
  if (!items || !q_ptr || !wk || !wv || !out || !q_strides || !w_strides || !out_strides || !kv_strides)
    return fail(BD_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (kv_max > 0 && (!table || !kv_k || !kv_v)) return fail(BD_ERR_INVALID_ARG, "%s: null page table or store", fn);
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return fail(BD_ERR_INVALID_ARG, "%s: bad sm_scale", fn);
  if (!strides_ok(kv_strides, 3, es) || !strides_ok(q_strides, 3, es) || !strides_ok(w_strides, 3, es) ||
      !strides_ok(out_strides, 3, es))
    return fail(BD_ERR_INVALID_ARG, "%s: strides must be >= 0 and 16-byte multiples", fn);
  if (!aligned16(q_ptr) || !aligned16(wk) || !aligned16(wv) || !aligned16(out) ||
      (kv_max > 0 && (!aligned16(kv_k) || !aligned16(kv_v))) || ((uintptr_t)items & 3u) != 0)
    return fail(BD_ERR_INVALID_ARG, "%s: base pointers must be 16-byte aligned", fn);
  if (kv_strides[1] * es * 64 > INT32_MAX || w_strides[1] * es * 64 > INT32_MAX)
    return fail(BD_ERR_INVALID_ARG, "%s: key row strides above 32 MB are not supported", fn);
  if ((int64_t)n_table * 4 > INT32_MAX) return fail(BD_ERR_INVALID_ARG, "%s: page table too long", fn);
  const AttnPlan plan = attn_plan(dtype, B, Hq, Hkv, d, q, n_items, kv_max, true);
  const int64_t grid_units = (8 + (int64_t)n_items * Hkv) * plan.nqt * plan.n_split;
  if (grid_units > ((int64_t)1 << 31) - 1)
    return fail(BD_ERR_INVALID_ARG, "%s: problem too large for one launch", fn);
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.dtype = dtype; a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.d = d; a.q = q; a.bl = bl;
  a.mask_mode = BD_MASK_BLOCK_CAUSAL;
  a.n_rows = n_items; a.n_rows1 = n_items;
  a.Q = q_ptr; a.wk = wk; a.wv = wv; a.out = out; a.lse = lse;
  memcpy(a.qs, q_strides, sizeof(a.qs));
  memcpy(a.ws, w_strides, sizeof(a.ws));
  memcpy(a.os, out_strides, sizeof(a.os));
  a.pk = kv_k; a.pv = kv_v; memcpy(a.ps, kv_strides, sizeof(a.ps));
  a.p_cap = n_pages; a.p_max = kv_max;
  a.items = items; a.table = table; a.n_table = n_table; a.page = page;
  a.scale2 = sm_scale * kLog2e;
  a.nw = plan.nw; a.nqt = plan.nqt; a.chunk = plan.chunk; a.n_split = plan.n_split;
  if (plan.ws_bytes > 0) {
    if (!workspace || ws_bytes < plan.ws_bytes)
      return fail(BD_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, plan.ws_bytes);
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(BD_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    attn_bind_workspace(a, plan, (char *)workspace);
  }
  return hip_status(launch_attn(a, (hipStream_t)stream), fn);
}

int bd_qkv_rope_write(int dtype, int B, int q, int Dm, int Hq, int Hkv, int d, const void *x,
                      const int64_t x_strides[2], const void *w, const int32_t *rope_pos,
                      float rope_base, void *q_out, const int64_t q_strides[3], void *k_cache,
                      void *v_cache, const int64_t c_strides[3], int c_cap, const int32_t *dst_pos,
                      void *stream) {
  g_err[0] = 0;
  if (dtype != BD_BF16) return fail(BD_ERR_UNSUPPORTED, "bd_qkv_rope_write: only BD_BF16 is built");
  if (d != 128) return fail(BD_ERR_UNSUPPORTED, "bd_qkv_rope_write: only d == 128 is built");
  if (B < 0 || q < 0 || Dm <= 0 || Hq <= 0 || Hkv <= 0 || c_cap < 0)
    return fail(BD_ERR_INVALID_ARG, "bd_qkv_rope_write: negative or zero size");
  if (Dm % 64 != 0) return fail(BD_ERR_UNSUPPORTED, "bd_qkv_rope_write: Dm must be a multiple of 64");
  if (!(rope_base > 1.f) || rope_base > 1e30f)
    return fail(BD_ERR_INVALID_ARG, "bd_qkv_rope_write: rope_base must be > 1");
  if ((int64_t)B * q > ((int64_t)1 << 24) || Hq + 2 * Hkv > 65535 ||
      cdiv(Hq + 2 * Hkv, 2) * cdiv((int64_t)B * q, 256) > INT32_MAX)
    return fail(BD_ERR_INVALID_ARG, "bd_qkv_rope_write: too large for one launch");
  if (B == 0 || q == 0) return BD_OK;
  if (!x || !w || !rope_pos || !q_out || !k_cache || !v_cache || !dst_pos || !x_strides ||
      !q_strides || !c_strides)
    return fail(BD_ERR_INVALID_ARG, "bd_qkv_rope_write: null pointer");
  if (!strides_ok(x_strides, 2, 2) || !strides_ok(q_strides, 3, 2) || !strides_ok(c_strides, 3, 2))
    return fail(BD_ERR_INVALID_ARG, "bd_qkv_rope_write: strides must be >= 0 and 16-byte multiples");
  if (!aligned16(x) || !aligned16(w) || !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(BD_ERR_INVALID_ARG, "bd_qkv_rope_write: base pointers must be 16-byte aligned");
  // the kernel addresses W and x with 32-bit byte offsets from their bases
  const int64_t w_bytes = (int64_t)(Hq + 2 * Hkv) * d * Dm * 2;
  const int64_t x_bytes = ((int64_t)(B - 1) * x_strides[0] + (int64_t)(q - 1) * x_strides[1] + Dm) * 2;
  if (w_bytes >= ((int64_t)1 << 31) || x_bytes >= ((int64_t)1 << 31))
    return fail(BD_ERR_UNSUPPORTED, "bd_qkv_rope_write: W and x must each span less than 2 GiB");
  ProduceArgs a;
  a.B = B; a.q = q; a.Dm = Dm; a.Hq = Hq; a.Hkv = Hkv; a.c_cap = c_cap;
  a.x = (const bf16 *)x; a.xs[0] = x_strides[0]; a.xs[1] = x_strides[1];
  a.w = (const bf16 *)w; a.rope_pos = rope_pos; a.dst_pos = dst_pos;
  for (int j = 0; j < 64; ++j) a.inv_freq[j] = pow((double)rope_base, -2.0 * j / 128.0);
  a.qo = (bf16 *)q_out; memcpy(a.qos, q_strides, sizeof(a.qos));
  a.kc = (bf16 *)k_cache; a.vc = (bf16 *)v_cache; memcpy(a.cs, c_strides, sizeof(a.cs));
  return hip_status(launch_produce(a, (hipStream_t)stream), "bd_qkv_rope_write launch");
}

int bd_check_attn(int B, const int32_t *row_ids, int n_rows, const int32_t *p_len, int p_max, int p_cap,
                  int p_hi, uint32_t *status, void *stream) {
  g_err[0] = 0;
  if (B < 0 || n_rows < 0 || p_max < 0 || p_cap < 0 || p_hi < 0)
    return fail(BD_ERR_INVALID_ARG, "bd_check_attn: negative size");
  if (!row_ids && n_rows > B) return fail(BD_ERR_INVALID_ARG, "bd_check_attn: n_rows > B without row_ids");
  if (n_rows == 0) return BD_OK;
  if (!status || !p_len) return fail(BD_ERR_INVALID_ARG, "bd_check_attn: null pointer");
  const int hi = p_max < p_cap ? (p_max < p_hi ? p_max : p_hi) : (p_cap < p_hi ? p_cap : p_hi);
  return hip_status(launch_check_attn(B, row_ids, n_rows, p_len, hi, status, (hipStream_t)stream),
                    "bd_check_attn launch");
}

int bd_check_scatter(int B, int q, int t, int data_cap, const int32_t *o, const int32_t *row_ids,
                     int n_rows, int aliased, uint32_t *status, void *stream) {
  g_err[0] = 0;
  if (B < 0 || q < 0 || t < 0 || data_cap < 0 || n_rows < 0)
    return fail(BD_ERR_INVALID_ARG, "bd_check_scatter: negative size");
  if (!row_ids && n_rows > B) return fail(BD_ERR_INVALID_ARG, "bd_check_scatter: n_rows > B without row_ids");
  if (n_rows == 0) return BD_OK;
  if (!status || !o) return fail(BD_ERR_INVALID_ARG, "bd_check_scatter: null pointer");
  return hip_status(launch_check_scatter(B, q, t, data_cap, o, row_ids, n_rows, aliased, status,
                                         (hipStream_t)stream),
                    "bd_check_scatter launch");
}

int bd_check_gather(int B, int Hkv, const int32_t *idx, int k_max, const int32_t *k_cnt, int src_cap,
                    uint32_t *status, void *stream) {
  g_err[0] = 0;
  if (B < 0 || Hkv <= 0 || k_max < 0 || src_cap < 0)
    return fail(BD_ERR_INVALID_ARG, "bd_check_gather: negative or zero size");
  if ((int64_t)B * Hkv > 65535) return fail(BD_ERR_INVALID_ARG, "bd_check_gather: B * Hkv too large");
  if (B == 0 || k_max == 0) return BD_OK;
  if (!status || !idx || !k_cnt) return fail(BD_ERR_INVALID_ARG, "bd_check_gather: null pointer");
  return hip_status(launch_check_gather(B, Hkv, idx, k_max, k_cnt, src_cap, status, (hipStream_t)stream),
                    "bd_check_gather launch");
}

int bd_check_select(int B, const int32_t *s_len, int s_max, int k_cap, const int32_t *k_sel, int k_max,
                    uint32_t *status, void *stream) {
  g_err[0] = 0;
  if (B < 0 || s_max < 0 || k_cap < 0 || k_max < 0)
    return fail(BD_ERR_INVALID_ARG, "bd_check_select: negative size");
  if (B == 0) return BD_OK;
  if (!status || !s_len || !k_sel) return fail(BD_ERR_INVALID_ARG, "bd_check_select: null pointer");
  return hip_status(launch_check_select(B, s_len, s_max < k_cap ? s_max : k_cap, k_sel, k_max, status,
                                        (hipStream_t)stream),
                    "bd_check_select launch");
}

int bd_check_block_table(int B, int q, const bd_attn_item *items, int n_items, const int32_t *table,
                         int n_table, int n_pages, int page, int kv_max, uint32_t *status, void *stream) {
  g_err[0] = 0;
  if (B < 0 || q < 0 || n_items < 0 || n_table < 0 || n_pages < 0 || kv_max < 0)
    return fail(BD_ERR_INVALID_ARG, "bd_check_block_table: negative size");
  if (page <= 0 || page % 64 != 0)
    return fail(BD_ERR_INVALID_ARG, "bd_check_block_table: page %d must be a positive multiple of 64", page);
  if (n_items == 0) return BD_OK;
  if (!status || !items || (n_table > 0 && !table))
    return fail(BD_ERR_INVALID_ARG, "bd_check_block_table: null pointer");
  return hip_status(launch_check_table(B, q, items, n_items, table, n_table, n_pages, page, kv_max, status,
                                       (hipStream_t)stream),
                    "bd_check_block_table launch");
}

int bd_mask_materialize(int B, int C, int q, int bl, int mask_mode, const int32_t *o, uint8_t *out,
                        void *stream) {
  g_err[0] = 0;
  if (B < 0 || C < 0 || q < 0 || bl <= 0 || q > C)
    return fail(BD_ERR_INVALID_ARG, "bd_mask_materialize: bad sizes");
  if (mask_mode != BD_MASK_BLOCK_CAUSAL && mask_mode != BD_MASK_ISOLATED && mask_mode != BD_MASK_SHARED_FIRST)
    return fail(BD_ERR_INVALID_ARG, "bd_mask_materialize: unknown mask mode %d", mask_mode);
  if (B == 0 || C == 0 || q == 0) return BD_OK;
  if (!o || !out) return fail(BD_ERR_INVALID_ARG, "bd_mask_materialize: null pointer");
  if (B > 65535 || q > 65535) return fail(BD_ERR_INVALID_ARG, "bd_mask_materialize: too large");
  return hip_status(launch_mask(B, C, q, bl, mask_mode, o, out, (hipStream_t)stream), "bd_mask_materialize launch");
}

}  // extern "C"
