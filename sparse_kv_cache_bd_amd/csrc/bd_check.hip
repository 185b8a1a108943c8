// Device check mode: the per-row values that live in device memory (row
// ids, lengths, offsets, gather indices, page tables) are compared with the
// contract of each operation, and a status word collects one bit per kind
// of violation.  The operations themselves never access memory out of
// bounds on such values (they clamp or skip, as the header states); these
// kernels let a caller learn that a row was clamped or skipped.
//
// Each kernel ORs bits into *status with one atomic per wave that found a
// violation; it never clears the word (the caller does, so several checks
// can accumulate into one word).
#include "bd_common.h"

namespace bd {
namespace {

constexpr int kThreads = 256;

// OR `bits` into *status: one atomic per wave (lanes' bits combined first).
__device__ inline void report(uint32_t *status, uint32_t bits) {
  uint32_t all = bits;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) all |= __shfl_xor(all, o);
  if (all != 0 && (threadIdx.x & 63) == 0) atomicOr(status, all);
}

__device__ inline bool outside(int v, int lo, int hi) { return v < lo || v > hi; }

// One thread per listed row.
__global__ __launch_bounds__(kThreads) void check_attn_kernel(int B, const int32_t *row_ids, int n_rows,
                                                              const int32_t *p_len, int p_hi,
                                                              uint32_t *status) {
  const int r = blockIdx.x * kThreads + threadIdx.x;
  uint32_t bits = 0;
  if (r < n_rows) {
    const int b = row_ids ? row_ids[r] : r;
    if (b < 0 || b >= B) bits |= BD_CHECK_ROW;
    else if (outside(p_len[b], 0, p_hi)) bits |= BD_CHECK_LENGTH;
  }
  report(status, bits);
}

__global__ __launch_bounds__(kThreads) void check_scatter_kernel(int B, int q, int t, int data_cap,
                                                                 const int32_t *o, const int32_t *row_ids,
                                                                 int n_rows, int aliased, uint32_t *status) {
  const int r = blockIdx.x * kThreads + threadIdx.x;
  uint32_t bits = 0;
  if (r < n_rows) {
    const int b = row_ids ? row_ids[r] : r;
    if (b < 0 || b >= B) {
      bits |= BD_CHECK_ROW;
    } else {
      const int ob = o[b];
      if (ob < 0 || (int64_t)ob + q > data_cap) bits |= BD_CHECK_OFFSET;
      else if (aliased && !((int64_t)ob + q <= t || ob == t)) bits |= BD_CHECK_ALIAS;
    }
  }
  report(status, bits);
}

// Block = (256 pool slots, row x KV head): the row's k_cnt and the indices
// of the slots the gather copies.
__global__ __launch_bounds__(kThreads) void check_gather_kernel(int Hkv, const int32_t *idx, int k_max,
                                                                const int32_t *k_cnt, int src_cap,
                                                                uint32_t *status) {
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int j = blockIdx.x * kThreads + threadIdx.x;
  const int cnt = k_cnt[b];
  uint32_t bits = 0;
  if (outside(cnt, 0, k_max) && j == 0 && bh % Hkv == 0) bits |= BD_CHECK_LENGTH;
  // the slots the gather copies: the first clamp(k_cnt, 0, k_max)
  if (j < clampi(cnt, 0, k_max)) {
    const int s = idx[(int64_t)bh * k_max + j];
    if (s < 0 || s >= src_cap) bits |= BD_CHECK_INDEX;
  }
  report(status, bits);
}

__global__ __launch_bounds__(kThreads) void check_select_kernel(int B, const int32_t *s_len, int s_hi,
                                                                const int32_t *k_sel, int k_max,
                                                                uint32_t *status) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  uint32_t bits = 0;
  if (b < B && (outside(s_len[b], 0, s_hi) || outside(k_sel[b], 0, k_max))) bits |= BD_CHECK_LENGTH;
  report(status, bits);
}

// Block = one item; its threads walk the item's page ids.
__global__ __launch_bounds__(kThreads) void check_table_kernel(int B, int q, const bd_attn_item *items,
                                                               const int32_t *table, int n_table,
                                                               int n_pages, int page, int kv_max,
                                                               uint32_t *status) {
  const bd_attn_item e = items[blockIdx.x];
  uint32_t bits = 0;
  bool pages = true;
  if (threadIdx.x == 0) {
    if (e.row < 0 || e.row >= B) bits |= BD_CHECK_ROW;
    if (e.q_begin < 0 || e.q_begin >= q || e.q_end <= e.q_begin) bits |= BD_CHECK_QUERIES;
    if (outside(e.kv_len, 0, kv_max)) bits |= BD_CHECK_LENGTH;
  }
  const int L = clampi(e.kv_len, 0, kv_max);
  const int64_t np = cdiv(L, page);
  if (e.table_off < 0 || (int64_t)e.table_off + np > n_table) {
    pages = false;
    if (threadIdx.x == 0) bits |= BD_CHECK_PAGE;
  }
  if (pages) {
    for (int64_t j = threadIdx.x; j < np; j += kThreads) {
      const int pg = table[e.table_off + j];
      if (pg < 0 || pg >= n_pages) bits |= BD_CHECK_PAGE;
    }
  }
  report(status, bits);
}

}  // namespace

hipError_t launch_check_attn(int B, const int32_t *row_ids, int n_rows, const int32_t *p_len, int p_hi,
                             uint32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(check_attn_kernel, dim3((unsigned)cdiv(n_rows, kThreads)), dim3(kThreads), 0, s, B,
                     row_ids, n_rows, p_len, p_hi, status);
  return hipGetLastError();
}

hipError_t launch_check_scatter(int B, int q, int t, int data_cap, const int32_t *o, const int32_t *row_ids,
                                int n_rows, int aliased, uint32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(check_scatter_kernel, dim3((unsigned)cdiv(n_rows, kThreads)), dim3(kThreads), 0, s, B,
                     q, t, data_cap, o, row_ids, n_rows, aliased, status);
  return hipGetLastError();
}

hipError_t launch_check_gather(int B, int Hkv, const int32_t *idx, int k_max, const int32_t *k_cnt,
                               int src_cap, uint32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(check_gather_kernel, dim3((unsigned)cdiv(k_max, kThreads), (unsigned)(B * Hkv)),
                     dim3(kThreads), 0, s, Hkv, idx, k_max, k_cnt, src_cap, status);
  return hipGetLastError();
}

hipError_t launch_check_select(int B, const int32_t *s_len, int s_hi, const int32_t *k_sel, int k_max,
                               uint32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(check_select_kernel, dim3((unsigned)cdiv(B, kThreads)), dim3(kThreads), 0, s, B, s_len,
                     s_hi, k_sel, k_max, status);
  return hipGetLastError();
}

hipError_t launch_check_table(int B, int q, const bd_attn_item *items, int n_items, const int32_t *table,
                              int n_table, int n_pages, int page, int kv_max, uint32_t *status,
                              hipStream_t s) {
  hipLaunchKernelGGL(check_table_kernel, dim3((unsigned)n_items), dim3(kThreads), 0, s, B, q, items, table,
                     n_table, n_pages, page, kv_max, status);
  return hipGetLastError();
}

}  // namespace bd
