// Representative-query selection (HERALD Sec. IV-A2, Sec. IV-B4).
//
// Pipeline (one stream, no host round trip):
//   prep   q_rep = mean (or one row) of the block queries, pre-scaled by
//          sm_scale*log2(e) and split into bf16 hi + lo parts; clears the
//          top-k state of the active rows.
//   scan   z[hq, s] = <q_rep[hq], K[s, h]> for s < S_b, streaming the K cache
//          once in coalesced 16-byte loads.  The G query heads of a KV head
//          are the rows of one v_mfma_f32_16x16x32_bf16 tile (q_rep hi and lo
//          accumulate into the same fp32 result, so the query keeps ~16
//          mantissa bits while K stays bf16).  Per-chunk running (max, sum);
//          the last chunk of a row to finish merges them (fixed order).
//   score  s_hat[h, s] = sum_g exp2(z[g, s] - m_g) / l_g, written once: these
//          are exactly the values that get ranked.
//   hist x3  exact radix select of the k-th largest score on its fp32 bit
//          pattern (non-negative floats order like their bit patterns),
//          digits of 11/11/10 bits; block histograms in LDS, merged with
//          global atomics; the last block of a pass picks the digit.
//   count, write  ordered stream compaction: every score above the threshold
//          plus the lowest-index ties, written in ascending position order,
//          then -1 padding.
#include "bd_common.h"

namespace bd {

namespace {

constexpr int kSD = 128;     // head dim of the selection path
constexpr int kTS = 256;     // tokens per scan block
constexpr int kCK = 4096;    // scores per top-k block
constexpr int kBins = 2048;  // radix digit bins (11 bits)
constexpr int kThreads = 256;

struct SelLayout {
  size_t qhi, qlo, z, part, stats, rowtick, scores, hist, tick, state, ccount, total;
  int nch_scan, nch_topk;
};

SelLayout sel_layout(int B, int Hq, int Hkv, int d, int s_max) {
  SelLayout L;
  L.nch_scan = (int)cdiv(s_max > 0 ? s_max : 1, kTS);
  L.nch_topk = (int)cdiv(s_max > 0 ? s_max : 1, kCK);
  const size_t P = (size_t)B * Hkv;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  L.qhi = take((size_t)B * Hq * d * 2);
  L.qlo = take((size_t)B * Hq * d * 2);
  L.z = take((size_t)B * Hq * (size_t)s_max * 4);
  L.part = take((size_t)B * Hq * L.nch_scan * 2 * 4);
  L.stats = take((size_t)B * Hq * 2 * 4);
  L.rowtick = take((size_t)B * 4);
  L.scores = take(P * (size_t)s_max * 4);
  L.hist = take(P * 3 * kBins * 4);
  L.tick = take(P * 4 * 4);
  L.state = take(P * 4 * 4);
  L.ccount = take(P * L.nch_topk * 2 * 4);
  L.total = off;
  return L;
}

struct SelPtrs {
  bf16 *qhi, *qlo;
  float *z, *part, *stats, *scores;
  uint32_t *rowtick, *hist, *tick, *state, *ccount;
  int nch_scan, nch_topk;
};

__device__ inline void row_sizes(const SelectArgs &a, int b, int &S, int &kb) {
  S = clampi(a.s_len[b], 0, min(a.s_max, a.k_cap));
  kb = clampi(a.k_sel[b], 0, a.k_max);
}

// Block-wide exclusive prefix sum over 256 threads (4 waves).
__device__ inline int block_excl_scan(int v, int *sh, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const int t = sh[w];
    if (w < wave) before += t;
    total += t;
  }
  return before + x - v;
}

// ------------------------------------------------------------------- prep
__global__ __launch_bounds__(kSD) void sel_prep_kernel(SelectArgs a, SelPtrs w) {
  const int hq = blockIdx.x, b = blockIdx.y;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0) return;
  const int d = threadIdx.x;
  const bf16 *qp = a.q + (int64_t)b * a.qs[0] + (int64_t)hq * a.qs[2] + d;
  float acc;
  if (a.rep_mode == BD_REP_ROW) {
    acc = (float)qp[(int64_t)a.rep_row * a.qs[1]];
  } else {
    acc = 0.f;
    for (int i = 0; i < a.nq; ++i) acc += (float)qp[(int64_t)i * a.qs[1]];
    acc /= (float)a.nq;
  }
  const float v = acc * a.scale2;
  const bf16 hi = (bf16)v;
  const bf16 lo = (bf16)(v - (float)hi);
  w.qhi[((int64_t)b * a.Hq + hq) * kSD + d] = hi;
  w.qlo[((int64_t)b * a.Hq + hq) * kSD + d] = lo;
  // clear the per-row ticket and the top-k state of this row's KV heads
  if (hq == 0 && d == 0) w.rowtick[b] = 0;
  const int words = a.Hkv * 3 * kBins;
  uint32_t *hist = w.hist + (size_t)b * words;
  for (int e = hq * kSD + d; e < words; e += a.Hq * kSD) hist[e] = 0;
  if (hq == 0 && d < a.Hkv) {
    const size_t p = (size_t)b * a.Hkv + d;
    for (int e = 0; e < 4; ++e) w.tick[p * 4 + e] = 0;
    w.state[p * 4 + 0] = 0;                 // threshold prefix
    w.state[p * 4 + 1] = (uint32_t)min(kb, S);  // remaining rank inside the prefix
    w.state[p * 4 + 2] = 0;
    w.state[p * 4 + 3] = 0;
  }
}

// ------------------------------------------------------------------- scan
__global__ __launch_bounds__(kThreads) void sel_scan_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, b = blockIdx.y;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0) return;
  const int nch = (int)cdiv(S, kTS);
  if (c >= nch) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15;   // token column of the 16x16 tile
  const int grp = lane >> 4;   // k-group (A/B operands) and row group (C)
  const int G = a.G;
  const int s0 = c * kTS;
  __shared__ int sh_ticket;

  for (int h = wave; h < a.Hkv; h += kThreads / 64) {
    // A operands: row col = query head h*G + col (zero rows past G)
    bf16x8 ahi[kSD / 32], alo[kSD / 32];
    {
      const bool ok = col < G;
      const bf16 *ph = w.qhi + ((int64_t)b * a.Hq + h * G + (ok ? col : 0)) * kSD + grp * 8;
      const bf16 *pl = w.qlo + ((int64_t)b * a.Hq + h * G + (ok ? col : 0)) * kSD + grp * 8;
#pragma unroll
      for (int ks = 0; ks < kSD / 32; ++ks) {
        ahi[ks] = ok ? *reinterpret_cast<const bf16x8 *>(ph + ks * 32) : bf16x8{};
        alo[ks] = ok ? *reinterpret_cast<const bf16x8 *>(pl + ks * 32) : bf16x8{};
      }
    }
    float m[4], l[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) { m[r] = -INFINITY; l[r] = 0.f; }
    const bf16 *kbase = a.k + (int64_t)b * a.ks[0] + (int64_t)h * a.ks[2] + grp * 8;

    for (int g16 = 0; g16 < kTS / 16; g16 += 2) {
      bf16x8 bop[2][kSD / 32];
      int tok[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        tok[j] = s0 + (g16 + j) * 16 + col;
        const bool ok = tok[j] < S;
        const bf16 *kp = kbase + (int64_t)(ok ? tok[j] : 0) * a.ks[1];
#pragma unroll
        for (int ks = 0; ks < kSD / 32; ++ks)
          bop[j][ks] = ok ? *reinterpret_cast<const bf16x8 *>(kp + ks * 32) : bf16x8{};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kSD / 32; ++ks) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[ks], bop[j][ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[ks], bop[j][ks], acc, 0, 0, 0);
        }
        if (tok[j] < S) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = grp * 4 + r;
            if (row < G) {
              const float z = acc[r];
              w.z[((int64_t)b * a.Hq + h * G + row) * a.s_max + tok[j]] = z;
              const float mn = fmaxf(m[r], z);
              l[r] = l[r] * __builtin_amdgcn_exp2f(m[r] - mn) + __builtin_amdgcn_exp2f(z - mn);
              m[r] = mn;
            }
          }
        }
      }
    }
    // merge (m, l) over the 16 token columns of each row group
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mo = __shfl_xor(m[r], o);
        const float lo = __shfl_xor(l[r], o);
        const float mn = fmaxf(m[r], mo);
        if (mn == -INFINITY) continue;
        l[r] = l[r] * __builtin_amdgcn_exp2f(m[r] - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
        m[r] = mn;
      }
    }
    if (col == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = grp * 4 + r;
        if (row < G) {
          float *pp = w.part + (((int64_t)b * a.Hq + h * G + row) * w.nch_scan + c) * 2;
          pp[0] = m[r];
          pp[1] = l[r];
        }
      }
    }
  }

  // the last block of the row merges all chunk statistics
  __threadfence();
  __syncthreads();
  if (tid == 0) sh_ticket = (int)atomicAdd(&w.rowtick[b], 1u);
  __syncthreads();
  if (sh_ticket != nch - 1) return;
  __threadfence();
  const int sub = tid & 7;
  for (int hq = tid >> 3; hq < a.Hq; hq += kThreads / 8) {
    float M = -INFINITY, L = 0.f;
    for (int cc = sub; cc < nch; cc += 8) {
      const float *pp = w.part + (((int64_t)b * a.Hq + hq) * w.nch_scan + cc) * 2;
      const float mc = pp[0], lc = pp[1];
      const float mn = fmaxf(M, mc);
      if (mn == -INFINITY) continue;
      L = L * __builtin_amdgcn_exp2f(M - mn) + lc * __builtin_amdgcn_exp2f(mc - mn);
      M = mn;
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const float mo = __shfl_xor(M, o);
      const float lo = __shfl_xor(L, o);
      const float mn = fmaxf(M, mo);
      if (mn == -INFINITY) continue;
      L = L * __builtin_amdgcn_exp2f(M - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
      M = mn;
    }
    if (sub == 0) {
      w.stats[((int64_t)b * a.Hq + hq) * 2 + 0] = M;
      w.stats[((int64_t)b * a.Hq + hq) * 2 + 1] = L;
    }
  }
}

// ------------------------------------------------------------------ score
__global__ __launch_bounds__(kThreads) void sel_score_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, b = blockIdx.y;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0) return;
  if (c >= (int)cdiv(S, kTS)) return;
  __shared__ float sm[64], sil[64];
  for (int hq = threadIdx.x; hq < a.Hq; hq += kThreads) {
    sm[hq] = w.stats[((int64_t)b * a.Hq + hq) * 2 + 0];
    sil[hq] = 1.f / w.stats[((int64_t)b * a.Hq + hq) * 2 + 1];
  }
  __syncthreads();
  const int s = c * kTS + threadIdx.x;
  if (s >= S) return;
  for (int h = 0; h < a.Hkv; ++h) {
    float acc = 0.f;
    for (int g = 0; g < a.G; ++g) {
      const int hq = h * a.G + g;
      const float z = w.z[((int64_t)b * a.Hq + hq) * a.s_max + s];
      acc += __builtin_amdgcn_exp2f(z - sm[hq]) * sil[hq];
    }
    w.scores[((int64_t)b * a.Hkv + h) * a.s_max + s] = acc;
  }
}

// ---------------------------------------------------------------- top-k
template <int PASS>
__global__ __launch_bounds__(kThreads) void sel_hist_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, p = blockIdx.y;
  const int b = p / a.Hkv;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0) return;
  const int nch = (int)cdiv(S, kCK);
  if (c >= nch) return;
  constexpr int shift = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  constexpr uint32_t dmask = PASS == 2 ? 1023u : 2047u;
  const uint32_t prefix = w.state[p * 4 + 0];
  const uint32_t krem = w.state[p * 4 + 1];
  __shared__ uint32_t hist[kBins];
  __shared__ int sh[8];
  __shared__ int sh_ticket;
  for (int e = threadIdx.x; e < kBins; e += kThreads) hist[e] = 0;
  __syncthreads();
  const uint32_t *keys = reinterpret_cast<const uint32_t *>(w.scores) + (size_t)p * a.s_max;
  for (int e = 0; e < kCK / kThreads; ++e) {
    const int s = c * kCK + e * kThreads + threadIdx.x;
    if (s < S) {
      const uint32_t key = keys[s];
      bool match = true;
      if (PASS == 1) match = (key >> 21) == (prefix >> 21);
      if (PASS == 2) match = (key >> 10) == (prefix >> 10);
      if (match) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
  }
  __syncthreads();
  uint32_t *gh = w.hist + ((size_t)p * 3 + PASS) * kBins;
  for (int e = threadIdx.x; e < kBins; e += kThreads)
    if (hist[e]) atomicAdd(&gh[e], hist[e]);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sh_ticket = (int)atomicAdd(&w.tick[p * 4 + PASS], 1u);
  __syncthreads();
  if (sh_ticket != nch - 1) return;
  __threadfence();
  // last block: find digit D with count(> D) < krem <= count(>= D)
  constexpr int per = kBins / kThreads;  // 8 bins per thread, descending order
  const int hi_bin = kBins - 1 - threadIdx.x * per;
  uint32_t cnt[per];
  int tsum = 0;
#pragma unroll
  for (int e = 0; e < per; ++e) {
    cnt[e] = gh[hi_bin - e];
    tsum += (int)cnt[e];
  }
  int total;
  const int before = block_excl_scan(tsum, sh, total);
  if ((uint32_t)before < krem && krem <= (uint32_t)(before + tsum)) {
    uint32_t cum = (uint32_t)before;
#pragma unroll
    for (int e = 0; e < per; ++e) {
      if (cum + cnt[e] >= krem) {
        const uint32_t D = (uint32_t)(hi_bin - e);
        w.state[p * 4 + 0] = prefix | (D << shift);
        w.state[p * 4 + 1] = krem - cum;
        break;
      }
      cum += cnt[e];
    }
  }
}

__global__ __launch_bounds__(kThreads) void sel_count_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, p = blockIdx.y;
  const int b = p / a.Hkv;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0) return;
  if (c >= (int)cdiv(S, kCK)) return;
  const uint32_t thr = w.state[p * 4 + 0];
  const uint32_t *keys = reinterpret_cast<const uint32_t *>(w.scores) + (size_t)p * a.s_max;
  int gt = 0, eq = 0;
  for (int e = 0; e < kCK / kThreads; ++e) {
    const int s = c * kCK + e * kThreads + threadIdx.x;
    if (s < S) {
      const uint32_t key = keys[s];
      gt += key > thr;
      eq += key == thr;
    }
  }
  __shared__ int sh[8];
  int tg, te;
  block_excl_scan(gt, sh, tg);
  block_excl_scan(eq, sh, te);
  if (threadIdx.x == 0) {
    w.ccount[((size_t)p * w.nch_topk + c) * 2 + 0] = (uint32_t)tg;
    w.ccount[((size_t)p * w.nch_topk + c) * 2 + 1] = (uint32_t)te;
  }
}

__global__ __launch_bounds__(kThreads) void sel_write_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, p = blockIdx.y;
  const int b = p / a.Hkv;
  int S, kb;
  row_sizes(a, b, S, kb);
  const int keff = min(S, kb);
  int32_t *out = a.idx_out + (size_t)p * a.k_max;
  if (c == 0)
    for (int j = keff + threadIdx.x; j < a.k_max; j += kThreads) out[j] = -1;
  if (keff == 0) return;
  if (c >= (int)cdiv(S, kCK)) return;
  const uint32_t thr = w.state[p * 4 + 0];
  const int need_eq = (int)w.state[p * 4 + 1];
  __shared__ int sh[8];
  // selected before this chunk: all "greater" ones plus the first ties
  int gtb = 0, eqb = 0;
  for (int cc = threadIdx.x; cc < c; cc += kThreads) {
    gtb += (int)w.ccount[((size_t)p * w.nch_topk + cc) * 2 + 0];
    eqb += (int)w.ccount[((size_t)p * w.nch_topk + cc) * 2 + 1];
  }
  int gt_before, eq_before;
  block_excl_scan(gtb, sh, gt_before);
  block_excl_scan(eqb, sh, eq_before);
  // this thread's 16 consecutive positions
  constexpr int per = kCK / kThreads;
  const int s0 = c * kCK + threadIdx.x * per;
  const uint32_t *keys = reinterpret_cast<const uint32_t *>(w.scores) + (size_t)p * a.s_max;
  uint32_t kv[per];
  int n_eq = 0;
#pragma unroll
  for (int e = 0; e < per; ++e) {
    const int s = s0 + e;
    kv[e] = (s < S) ? keys[s] : 0u;
    n_eq += (s < S) && kv[e] == thr;
  }
  int tot;
  const int eq_rank0 = eq_before + block_excl_scan(n_eq, sh, tot);
  int n_sel = 0, er = eq_rank0;
  uint32_t selbits = 0;
#pragma unroll
  for (int e = 0; e < per; ++e) {
    const int s = s0 + e;
    bool sel = false;
    if (s < S) {
      if (kv[e] > thr) sel = true;
      else if (kv[e] == thr) { sel = er < need_eq; ++er; }
    }
    selbits |= (uint32_t)sel << e;
    n_sel += sel;
  }
  const int pos0 = gt_before + min(eq_before, need_eq) + block_excl_scan(n_sel, sh, tot);
  int pos = pos0;
#pragma unroll
  for (int e = 0; e < per; ++e)
    if (selbits & (1u << e)) {
      if (pos < keff) out[pos] = s0 + e;
      ++pos;
    }
}

}  // namespace

size_t select_workspace(int B, int Hq, int Hkv, int d, int s_max, int k_max) {
  (void)k_max;
  return sel_layout(B, Hq, Hkv, d, s_max).total;
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  const SelLayout L = sel_layout(a.B, a.Hq, a.Hkv, a.d, a.s_max);
  SelPtrs w;
  w.qhi = reinterpret_cast<bf16 *>(a.ws + L.qhi);
  w.qlo = reinterpret_cast<bf16 *>(a.ws + L.qlo);
  w.z = reinterpret_cast<float *>(a.ws + L.z);
  w.part = reinterpret_cast<float *>(a.ws + L.part);
  w.stats = reinterpret_cast<float *>(a.ws + L.stats);
  w.rowtick = reinterpret_cast<uint32_t *>(a.ws + L.rowtick);
  w.scores = a.score_out ? a.score_out : reinterpret_cast<float *>(a.ws + L.scores);
  w.hist = reinterpret_cast<uint32_t *>(a.ws + L.hist);
  w.tick = reinterpret_cast<uint32_t *>(a.ws + L.tick);
  w.state = reinterpret_cast<uint32_t *>(a.ws + L.state);
  w.ccount = reinterpret_cast<uint32_t *>(a.ws + L.ccount);
  w.nch_scan = L.nch_scan;
  w.nch_topk = L.nch_topk;
  hipError_t e;
  hipLaunchKernelGGL(sel_prep_kernel, dim3(a.Hq, a.B), dim3(kSD), 0, s, a, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sel_scan_kernel, dim3(L.nch_scan, a.B), dim3(kThreads), 0, s, a, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sel_score_kernel, dim3(L.nch_scan, a.B), dim3(kThreads), 0, s, a, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 tg(L.nch_topk, a.B * a.Hkv);
  hipLaunchKernelGGL(sel_hist_kernel<0>, tg, dim3(kThreads), 0, s, a, w);
  hipLaunchKernelGGL(sel_hist_kernel<1>, tg, dim3(kThreads), 0, s, a, w);
  hipLaunchKernelGGL(sel_hist_kernel<2>, tg, dim3(kThreads), 0, s, a, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sel_count_kernel, tg, dim3(kThreads), 0, s, a, w);
  hipLaunchKernelGGL(sel_write_kernel, tg, dim3(kThreads), 0, s, a, w);
  return hipGetLastError();
}

}  // namespace bd
