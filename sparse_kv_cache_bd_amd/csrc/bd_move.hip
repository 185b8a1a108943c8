// KV movement kernels: the write-back scatter (FlowBlock review Eq. (7)),
// the pool gather (HERALD Sec. IV-B3) and the mask test hook.
//
// Both copies are HBM-bound: every byte is read once and written once, in
// 16-byte vectors, with 16 consecutive lanes covering one 256-byte (pos,
// head) row so each wave instruction moves whole contiguous segments.
#include "bd_common.h"

namespace bd {

namespace {

constexpr int kThreads = 256;

__device__ inline uint4 ld16(const char *p) { return *reinterpret_cast<const uint4 *>(p); }
// Stores are nontemporal (streaming): the copies' destinations are not read
// again by the same launch, and the hint keeps them from displacing cached
// lines (the scatter's and gather's sources) on their way to HBM.
__device__ inline void st16(char *p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

// One block moves kTok window positions of one (layer, row, tensor) for all
// KV heads.  vpr = 16-byte vectors per (pos, head) row = d * es / 16.
constexpr int kTok = 16;
constexpr int kScatterUnroll = 8;

__global__ __launch_bounds__(kThreads) void scatter_kernel(ScatterArgs a, int vpr) {
  const int rl = blockIdx.y;
  const int layer = blockIdx.z >> 1;
  const int which = blockIdx.z & 1;  // 0 = K, 1 = V
  const char *src = which ? a.pv : a.pk;
  char *dst = which ? a.dv : a.dk;
  if (src == nullptr) return;
  const int b = a.row_ids ? a.row_ids[rl] : rl;
  if (b < 0 || b >= a.B) return;
  const int ob = a.o[b];
  if (ob < 0 || (int64_t)ob + a.q > a.data_cap) return;  // row skipped

  const int tok0 = blockIdx.x * kTok;
  const int ntok = min(kTok, a.q - tok0);
  const int per_tok = a.Hkv * vpr;
  const int total = ntok * per_tok;
  const char *sbase = src + ((int64_t)layer * a.ps[0] + (int64_t)b * a.ps[1]) * a.es;
  char *dbase = dst + ((int64_t)layer * a.ds[0] + (int64_t)b * a.ds[1]) * a.es;

  for (int e0 = threadIdx.x; e0 < total; e0 += kThreads * kScatterUnroll) {
    uint4 v[kScatterUnroll];
    int64_t doff[kScatterUnroll];
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
      const int e = e0 + u * kThreads;
      if (e < total) {
        const int tok = e / per_tok;
        const int rem = e - tok * per_tok;
        const int h = rem / vpr;
        const int c = rem - h * vpr;
        const int pos = tok0 + tok;
        v[u] = ld16(sbase + ((int64_t)(a.t + pos) * a.ps[2] + (int64_t)h * a.ps[3]) * a.es + c * 16);
        doff[u] = ((int64_t)(ob + pos) * a.ds[2] + (int64_t)h * a.ds[3]) * a.es + c * 16;
      }
    }
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
      const int e = e0 + u * kThreads;
      if (e < total) st16(dbase + doff[u], v[u]);
    }
  }
}

// One block gathers kSlots pool slots of one (row, KV head, tensor).
constexpr int kSlots = 64;

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a, int vpr) {
  const int bh = blockIdx.y;
  const int b = bh / a.Hkv;
  const int h = bh - b * a.Hkv;
  const int which = blockIdx.z;
  const char *src = which ? a.vs : a.ks;
  char *dst = which ? a.vp : a.kp;
  if (src == nullptr) return;
  const int cnt = clampi(a.k_cnt[b], 0, a.k_max);
  const int j0 = blockIdx.x * kSlots;
  if (j0 >= cnt) return;
  const int nslot = min(kSlots, cnt - j0);
  const int total = nslot * vpr;
  const int32_t *idx = a.idx + ((int64_t)b * a.Hkv + h) * a.k_max + j0;
  const char *sbase = src + ((int64_t)b * a.ss[0] + (int64_t)h * a.ss[2]) * a.es;
  char *dbase = dst + ((int64_t)b * a.pls[0] + (int64_t)h * a.pls[2]) * a.es;
  constexpr int U = 4;
  for (int e0 = threadIdx.x; e0 < total; e0 += kThreads * U) {
    uint4 v[U];
    int64_t doff[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * kThreads;
      ok[u] = false;
      if (e < total) {
        const int j = e / vpr;
        const int c = e - j * vpr;
        const int s = idx[j];
        if (s >= 0 && s < a.src_cap) {
          ok[u] = true;
          v[u] = ld16(sbase + (int64_t)s * a.ss[1] * a.es + c * 16);
          doff[u] = (int64_t)(j0 + j) * a.pls[1] * a.es + c * 16;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) st16(dbase + doff[u], v[u]);
  }
}

__global__ __launch_bounds__(kThreads) void mask_kernel(int B, int C, int q, int bl, int mode,
                                                        const int32_t *o, uint8_t *out) {
  const int b = blockIdx.z;
  const int i = blockIdx.y;
  const int j = blockIdx.x * kThreads + threadIdx.x;
  if (j >= C) return;
  const int t = C - q;
  const int ob = o[b];
  uint8_t v;
  if (ob < 0 || ob > t)
    v = 0xFF;
  else
    v = cache_visible(i, j, ob, t, bl, q, mode) ? 1 : 0;
  out[((int64_t)b * q + i) * C + j] = v;
}

}  // namespace

hipError_t launch_scatter(const ScatterArgs &a, hipStream_t s) {
  const int vpr = a.d * a.es / 16;
  dim3 grid((unsigned)cdiv(a.q, kTok), (unsigned)a.n_rows, (unsigned)(a.n_layers * 2));
  hipLaunchKernelGGL(scatter_kernel, grid, dim3(kThreads), 0, s, a, vpr);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
  const int vpr = a.d * a.es / 16;
  dim3 grid((unsigned)cdiv(a.k_max, kSlots), (unsigned)(a.B * a.Hkv), 2u);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(kThreads), 0, s, a, vpr);
  return hipGetLastError();
}

hipError_t launch_mask(int B, int C, int q, int bl, int mode, const int32_t *o, uint8_t *out,
                       hipStream_t s) {
  dim3 grid((unsigned)cdiv(C, kThreads), (unsigned)q, (unsigned)B);
  hipLaunchKernelGGL(mask_kernel, grid, dim3(kThreads), 0, s, B, C, q, bl, mode, o, out);
  return hipGetLastError();
}

}  // namespace bd
