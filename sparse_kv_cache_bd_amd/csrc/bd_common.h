// Internal definitions shared by the libbdattn sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bdattn.h"

namespace bd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Error reporting (thread-local message, defined in bd_api.hip).
void set_error(const char *fmt, ...);

// log2(e): the kernels evaluate exp(x) as exp2(x * log2(e)).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Visibility predicate of the per-row block-diagonal mask (FlowBlock review
// Eq. (6)).  In window coordinates a query i sees window keys w < lim(i),
// lim(i) = min(q, (floor(i/bl) + 1) * bl); every prefix key j < P_b is
// visible.  The attention kernels and the mask test hook both call these.
// ---------------------------------------------------------------------------
__host__ __device__ inline int window_limit(int i, int bl, int q) {
  int lim = (i / bl + 1) * bl;
  return lim < q ? lim : q;
}

// Other window masks (bd_mask_mode): query i sees window key w when
// w < window_limit(i) and (w < window_shared or w >= window_floor(i)): the
// block-causal mask has floor 0; isolated groups start at their own block;
// a shared first block stays visible to every group.
__host__ __device__ inline int window_floor(int i, int bl, int mode) {
  return mode == BD_MASK_BLOCK_CAUSAL ? 0 : (i / bl) * bl;
}
__host__ __device__ inline int window_shared(int bl, int mode) {
  return mode == BD_MASK_SHARED_FIRST ? bl : 0;
}

__host__ __device__ inline bool window_visible(int i, int w, int bl, int q, int mode) {
  return w < window_limit(i, bl, q) && (w < window_shared(bl, mode) || w >= window_floor(i, bl, mode));
}

__host__ __device__ inline bool cache_visible(int i, int j, int ob, int t, int bl, int q, int mode) {
  if (j < ob) return true;
  return j >= t && window_visible(i, j - t, bl, q, mode);
}

__host__ __device__ inline int clampi(int v, int lo, int hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Exchange with lane l ^ 32 (the other half of the wave).
__device__ inline float xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // lanes < 32 receive the upper half in r[1]; lanes >= 32 the lower half in r[0]
  return (__lane_id() < 32) ? __uint_as_float(r[1]) : __uint_as_float(r[0]);
}

// ---------------------------------------------------------------------------
// Kernel launchers (host side), one per operation.  Arguments are validated
// by the public entry points before these are called.
// ---------------------------------------------------------------------------
struct ScatterArgs {
  int es;  // element size in bytes
  int B, Hkv, d, q, n_layers, n_rows, t, present_cap, data_cap;
  const char *pk, *pv;
  char *dk, *dv;
  int64_t ps[4], ds[4];  // element strides {layer, row, pos, head}
  const int32_t *o, *row_ids;
};
hipError_t launch_scatter(const ScatterArgs &a, hipStream_t s);

struct GatherArgs {
  int es;
  int B, Hkv, d, src_cap, k_max, pool_cap;
  const char *ks, *vs;
  char *kp, *vp;
  int64_t ss[3], pls[3];
  const int32_t *idx, *k_cnt;
};
hipError_t launch_gather(const GatherArgs &a, hipStream_t s);

hipError_t launch_mask(int B, int C, int q, int bl, int mode, const int32_t *o, uint8_t *out,
                       hipStream_t s);

struct AttnArgs {
  int dtype;  // BD_BF16 / BD_F32
  int B, Hq, Hkv, G, d, q, bl, n_rows, p_cap, p_max;
  int mask_mode;  // bd_mask_mode of the window part
  const void *Q;
  int64_t qs[3];
  const void *pk, *pv;
  int64_t ps[3];
  const void *wk, *wv;
  int64_t ws[3];
  void *out;
  int64_t os[3];
  float *lse;
  const int32_t *row_ids, *p_len;
  // second prefix source (one launch over two row lists): list positions
  // at or past n_rows1 are rows row_ids2[pos - n_rows1] whose prefix is
  // pk2/pv2 with lengths p_len2.  A single-source call has n_rows1 = n_rows.
  int n_rows1;
  const int32_t *row_ids2, *p_len2;
  const void *pk2, *pv2;
  int64_t ps2[3];
  int p_cap2, p_max2;
  float scale2;  // sm_scale * log2(e)
  // block-table mode (bd_attn_block_table): the list positions are work
  // items {row, q_begin, q_end, table_off, kv_len} in the caller's order;
  // an item's keys are kv_len keys on the pages table[table_off ..] of the
  // paged store pk/pv (strides ps = {page, pos, head}; p_cap = pages).
  const bd_attn_item *items;
  const int32_t *table;
  int n_table, page;
  // launch plan (attn_plan)
  int nw;                 // waves per block of the MFMA path (4 or 8)
  int nqt, chunk, n_split;
  int *row_order;         // rows by descending prefix length, or NULL (natural order)
  bf16 *part_o;    // split partials: O / l of each chunk, bf16 (MFMA path)
  float *gpart_o;  // split partials: O / l of each chunk, fp32 (general path)
  float *part_ml;  // (max, sum) of each chunk
};
// Launch plan of one bd_attn_packed call: block shape, query tiles, key
// chunks per (row, KV head, query tile) unit, whether rows are ordered
// longest first, and the workspace this needs (offsets of its parts).
struct AttnPlan {
  int nw, nqt, chunk, n_split;
  bool order;
  size_t off_order, off_part_o, off_part_ml, ws_bytes;
};
AttnPlan attn_plan(int dtype, int B, int Hq, int Hkv, int d, int q, int n_rows, int p_max,
                   bool keep_order = false);
hipError_t launch_attn(const AttnArgs &a, hipStream_t s);

// One prefix source of an attention call: its row list and the prefix
// tensors those rows attend over.
struct PrefixArg {
  const int32_t *rows;
  int n;
  const void *pk, *pv;
  const int64_t *strides;
  int cap;
  const int32_t *p_len;
  int p_max;
};
// Validation (before any HIP call), argument block and plan of one
// attention call (bd_api.hip); *launch is false when there is nothing to do.
int attn_setup(const char *fn, int dtype, int B, int Hq, int Hkv, int d, int q, int bl,
               int mask_mode, const void *q_ptr, const int64_t q_strides[3], const PrefixArg &pa,
               const PrefixArg *pb, const void *wk, const void *wv, const int64_t w_strides[3],
               float sm_scale, void *out, const int64_t out_strides[3], float *lse,
               AttnArgs &a, AttnPlan &plan, bool *launch);
void attn_bind_workspace(AttnArgs &a, const AttnPlan &plan, char *ws);
// BD_OK, or BD_ERR_HIP with the message set.
int attn_launch_status(hipError_t e, const char *fn);
bool attn_mfma_supported(int dtype, int d, int G);
bool attn_generic_supported(int dtype, int d);

struct SelectArgs {
  int B, Hq, Hkv, G, d, nq, rep_mode, rep_row, k_cap, s_max, k_max;
  const bf16 *q;
  int64_t qs[3];
  const bf16 *k;
  int64_t ks[3];
  const int32_t *s_len, *k_sel;
  float scale2;
  int32_t *idx_out;
  float *score_out;
  char *ws;
  // representative query's attention output (bd_select_attn); null in bd_select
  const bf16 *v;
  int64_t vs[3];
  bf16 *o_rep;
};
size_t select_workspace(int B, int Hq, int Hkv, int d, int s_max, int k_max, bool with_out = false);
hipError_t launch_select(const SelectArgs &a, hipStream_t s);
// Exact multi-query selection: nq * G <= 128 columns per KV head.
size_t select_multi_workspace(int B, int Hkv, int s_max);
hipError_t launch_select_multi(const SelectArgs &a, hipStream_t s);

// Device check mode (bd_check.hip): OR BD_CHECK_* bits into *status.
hipError_t launch_check_attn(int B, const int32_t *row_ids, int n_rows, const int32_t *p_len, int p_hi,
                             uint32_t *status, hipStream_t s);
hipError_t launch_check_scatter(int B, int q, int t, int data_cap, const int32_t *o, const int32_t *row_ids,
                                int n_rows, int aliased, uint32_t *status, hipStream_t s);
hipError_t launch_check_gather(int B, int Hkv, const int32_t *idx, int k_max, const int32_t *k_cnt,
                               int src_cap, uint32_t *status, hipStream_t s);
hipError_t launch_check_select(int B, const int32_t *s_len, int s_hi, const int32_t *k_sel, int k_max,
                               uint32_t *status, hipStream_t s);
hipError_t launch_check_table(int B, int q, const bd_attn_item *items, int n_items, const int32_t *table,
                              int n_table, int n_pages, int page, int kv_max, uint32_t *status,
                              hipStream_t s);

// Fused cache producer: QKV projection + RoPE + cache write (d = 128, bf16).
struct ProduceArgs {
  int B, q, Dm, Hq, Hkv, c_cap;
  const bf16 *x;
  int64_t xs[2];            // {row, token}
  const bf16 *w;            // [(Hq + 2 Hkv) * 128, Dm], contiguous
  const int32_t *rope_pos;  // absolute position of window token 0, per row
  const int32_t *dst_pos;   // cache position of window token 0, per row
  double inv_freq[64];      // rope_base^(-2j/128), j < 64
  float step_rot[64][2];    // cos, sin of 32 x inv_freq[j] (set by launch_produce)
  bf16 *qo;
  int64_t qos[3];
  bf16 *kc, *vc;
  int64_t cs[3];
};
hipError_t launch_produce(const ProduceArgs &a, hipStream_t s);

}  // namespace bd
