// Representative-query selection (HERALD Sec. IV-A2, Sec. IV-B4).
//
// Four kernels on one stream, no host round trip:
//   prep   q_rep = mean (or one row) of the block queries, pre-scaled by
//          sm_scale*log2(e) and split into bf16 hi + lo parts.
//   scan   z[hq, s] = <q_rep[hq], K[s, h]> for s < S_b: streams the K cache
//          once with 16-byte loads; the loads of the next two 64-token
//          groups are in flight while the current group is computed.  Tokens are the
//          rows of v_mfma_f32_16x16x32_bf16 and the G query heads of a KV
//          head its columns (q_rep hi and lo accumulate into the same fp32
//          result, so the query keeps ~16 mantissa bits while K stays bf16);
//          a lane then holds 4 consecutive tokens of one head.  z of the
//          block's chunk is staged in LDS and written with coalesced 16-byte
//          stores after the loop (stores share the load counter, so none are
//          issued while loads are in flight).  Per-block running (max, sum)
//          per query head.
//   score  m_g, l_g = fixed-order merge of the scan's per-block (max, sum);
//          s_hat[h, s] = sum_g exp2(z[g, s] - m_g) / l_g, written once: these
//          are exactly the values that get ranked.  (No cross-block merge
//          inside the scan: that needs device-scope fences, which write back
//          and invalidate the L2 of the XCD on every block.)
//   out    (bd_select_attn only) the representative query's attention
//          output, o[g] = sum_s exp2(z[g, s] - m_g) / l_g * V[s]: a pass
//          over V after the score pass with the same weights, fp32 partials
//          per 1024-token chunk, summed in chunk order by a merge kernel.
//   topk   exact radix select of the k-th largest score on its fp32 bit
//          pattern (non-negative floats order like their bit patterns;
//          digits of 11, 11 and 10 bits; the first digit's histogram is
//          built by the score pass), then an ordered compaction: every
//          score above the threshold plus the lowest-position ties,
//          ascending, -1 padding (one prefix sum per chunk when every tie is
//          kept).  Rows of up to kLdsKeys scores: one block
//          per (row, KV head) with the scores read once into LDS.  Longer
//          rows: blocks of kCK scores; the score pass histograms the first
//          digit, two passes the others, then per-block counts and an
//          ordered write.
//
// Histogram increments are aggregated per wave: lanes whose digit equals the
// first active lane's digit add in one atomic (two rounds), so the strongly
// clustered digits of softmax-like scores do not serialise on one LDS bank.
#include "bd_common.h"

namespace bd {

namespace {

constexpr int kSD = 128;           // head dim of the selection path
constexpr int kTS = 256;           // tokens per scan block
constexpr int kScoreTok = 1024;    // tokens per score block
constexpr int kBins = 2048;        // radix digit bins (11 bits)
constexpr int kThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kPerThread = 16;     // consecutive scores per thread in the compaction
constexpr int kRankU = 8;          // keys per thread per histogram round
constexpr int kLdsKeys = 32768;    // longest score row ranked by one block from LDS
constexpr int kCK = 4096;          // scores per block of the multi-block ranking path
constexpr int kZStr = kTS + 16;    // LDS row stride of the scan's z staging (floats)
constexpr int kOTok = 1024;        // tokens per block of the output pass

struct SelLayout {
  size_t qhi, qlo, z, part, scores, hist, ccount, opart, total;
  int nch_scan, nch_topk, nch_o;
  bool multi;  // rows longer than kLdsKeys: multi-block ranking
  int zs;  // row stride of z (s_max rounded up to 4: 16-byte aligned rows)
};

SelLayout sel_layout(int B, int Hq, int Hkv, int d, int s_max, bool with_out = false) {
  SelLayout L;
  L.nch_scan = (int)cdiv(s_max > 0 ? s_max : 1, kTS);
  L.nch_topk = (int)cdiv(s_max > 0 ? s_max : 1, kCK);
  L.nch_o = (int)cdiv(s_max > 0 ? s_max : 1, kOTok);
  L.multi = s_max > kLdsKeys;
  L.zs = (int)cdiv(s_max, 4) * 4;
  const size_t P = (size_t)B * Hkv;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  L.qhi = take((size_t)B * Hq * d * 2);
  L.qlo = take((size_t)B * Hq * d * 2);
  L.z = take((size_t)B * Hq * (size_t)L.zs * 4);
  L.part = take((size_t)B * Hq * L.nch_scan * 2 * 4);
  L.scores = take(P * (size_t)s_max * 4);
  L.hist = take(P * 3 * kBins * 4);
  L.ccount = L.multi ? take(P * L.nch_topk * 2 * 4) : 0;
  L.opart = with_out ? take(P * L.nch_o * (size_t)(Hq / Hkv) * d * 4) : 0;
  L.total = off;
  return L;
}

struct SelPtrs {
  bf16 *qhi, *qlo;
  float *z, *part, *scores;
  uint32_t *hist, *ccount;   // digit histograms (digit 0 for every row); per-chunk counts
  float *opart;              // output pass: fp32 partials [row][KV head][chunk][G][d]
  int nch_scan, zs, nch_topk, nch_o;
  bool multi;
};

__device__ inline void row_sizes(const SelectArgs &a, int b, int &S, int &kb) {
  S = clampi(a.s_len[b], 0, min(a.s_max, a.k_cap));
  kb = clampi(a.k_sel[b], 0, a.k_max);
}

// Merge running (max, sum) pairs in log2 units.
__device__ inline void merge_ml(float &m, float &l, float mo, float lo) {
  const float mn = fmaxf(m, mo);
  if (mn == -INFINITY) return;
  l = l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
  m = mn;
}

// Block-wide exclusive prefix sum (any multiple of 64 threads, <= 1024).
// sh holds at least 16 ints.
__device__ inline int block_excl_scan(int v, int *sh, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
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
  for (int w = 0; w < nw; ++w) {
    const int t = sh[w];
    if (w < wave) before += t;
    total += t;
  }
  return before + x - v;
}

// Histogram increment for one key per lane (valid lanes only): two rounds of
// per-wave aggregation of the most common digit, then single increments.
__device__ inline void hist_add(uint32_t *h, uint32_t bin, bool valid) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const uint64_t act = __ballot(valid);
    if (act == 0) return;
    const int leader = __builtin_ctzll(act);
    const uint32_t b0 = __builtin_amdgcn_readlane(bin, leader);
    const uint64_t same = __ballot(valid && bin == b0);
    if (lane == leader) atomicAdd(&h[b0], (uint32_t)__builtin_popcountll(same));
    if (bin == b0) valid = false;
  }
  if (valid) atomicAdd(&h[bin], 1u);
}

// ------------------------------------------------------------------- prep
// Block = (query head, row), 256 threads: thread t sums queries i = t/16,
// t/16 + 16, ... over dims 8*(t%16) .. +8 (16-byte loads), then the 16
// partial sums of each dim chunk are added in a fixed order.
__global__ __launch_bounds__(kThreads) void sel_prep_kernel(SelectArgs a, SelPtrs w) {
  const int hq = blockIdx.x, b = blockIdx.y;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0) return;
  const int t = threadIdx.x, dc = t & 15, qs = t >> 4;
  const bf16 *qp = a.q + (int64_t)b * a.qs[0] + (int64_t)hq * a.qs[2] + dc * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (a.rep_mode == BD_REP_ROW) {
    if (qs == 0) {
      const bf16x8 v = *reinterpret_cast<const bf16x8 *>(qp + (int64_t)a.rep_row * a.qs[1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = (float)v[e];
    }
  } else {
    // 8 loads in flight per round; summed in query order
    for (int i0 = qs; i0 < a.nq; i0 += 16 * 8) {
      bf16x8 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + 16 * u;
        v[u] = i < a.nq ? *reinterpret_cast<const bf16x8 *>(qp + (int64_t)i * a.qs[1]) : bf16x8{};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + 16 * u < a.nq)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += (float)v[u][e];
    }
  }
  __shared__ float part[16][kSD + 4];
#pragma unroll
  for (int e = 0; e < 8; ++e) part[qs][dc * 8 + e] = acc[e];
  __syncthreads();
  if (t < kSD) {
    float sum = 0.f;
    for (int i = 0; i < 16; ++i) sum += part[i][t];
    if (a.rep_mode != BD_REP_ROW) sum /= (float)a.nq;
    const float v = sum * a.scale2;
    const bf16 hi = (bf16)v;
    const bf16 lo = (bf16)(v - (float)hi);
    w.qhi[((int64_t)b * a.Hq + hq) * kSD + t] = hi;
    w.qlo[((int64_t)b * a.Hq + hq) * kSD + t] = lo;
  }
  {  // this row's digit histograms (Hkv x 3 x kBins words)
    const int words = a.Hkv * 3 * kBins;
    uint32_t *hist = w.hist + (size_t)b * words;
    for (int e = hq * kThreads + t; e < words; e += a.Hq * kThreads) hist[e] = 0;
  }
}

// ------------------------------------------------------------------- scan
// Block = (token chunk of kTS, row).  Wave w handles KV heads w, w+4, ...;
// its work is a flat list of (head, 64-token group) items.  The 16 loads of
// 16 bytes per lane of items i+1 and i+2 are in flight during item i.  The
// row's q_rep hi / lo parts are staged in LDS once per block.
__global__ __launch_bounds__(kThreads, 2) void sel_scan_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, b = blockIdx.y;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0) return;
  const int nch = (int)cdiv(S, kTS);
  if (c >= nch) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15;   // token row of the A operand; query head of B and C
  const int grp = lane >> 4;   // k-group of A/B; row group of C
  const int G = a.G;
  const int s0 = c * kTS;
  const int s_end = min(s0 + kTS, S);
  // dynamic LDS: q_rep hi and lo [Hq][kSD] bf16, then z of this chunk [Hq][kZStr] fp32
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16 *qs_hi = reinterpret_cast<bf16 *>(smem);
  bf16 *qs_lo = qs_hi + a.Hq * kSD;
  float *zs = reinterpret_cast<float *>(qs_lo + a.Hq * kSD);
  __shared__ float ml_lds[64][2];   // per query head (max, sum) of this chunk
  {
    const bf16x8 *gh = reinterpret_cast<const bf16x8 *>(w.qhi + (int64_t)b * a.Hq * kSD);
    const bf16x8 *gl = reinterpret_cast<const bf16x8 *>(w.qlo + (int64_t)b * a.Hq * kSD);
    for (int e = tid; e < a.Hq * kSD / 8; e += kThreads) {
      reinterpret_cast<bf16x8 *>(qs_hi)[e] = gh[e];
      reinterpret_cast<bf16x8 *>(qs_lo)[e] = gl[e];
    }
  }
  __syncthreads();

  const int n_groups = (int)cdiv(s_end - s0, 64);
  const int n_heads = a.Hkv > wave ? (int)cdiv(a.Hkv - wave, kThreads / 64) : 0;
  const int n_items = n_heads * n_groups;
  auto item_head = [&](int i) { return wave + (kThreads / 64) * (i / n_groups); };
  auto item_t0 = [&](int i) { return s0 + 64 * (i % n_groups); };

  bf16x8 abuf[3][4][kSD / 32];
  auto load = [&](int i, bf16x8 (&dst)[4][kSD / 32]) {
    const int h = item_head(i), t0 = item_t0(i);
    const bf16 *kbase = a.k + (int64_t)b * a.ks[0] + (int64_t)h * a.ks[2] + grp * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = min(t0 + 16 * j + col, S - 1);   // clamped rows are discarded below
      const bf16 *kp = kbase + (int64_t)tok * a.ks[1];
#pragma unroll
      for (int ks = 0; ks < kSD / 32; ++ks) dst[j][ks] = *reinterpret_cast<const bf16x8 *>(kp + ks * 32);
    }
  };

  float m = -INFINITY, l = 0.f;   // running stats of column col of the current head
  auto flush = [&](int h) {
    // merge over the 4 row groups holding the same column (lanes col + 16*grp)
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) merge_ml(m, l, __shfl_xor(m, o), __shfl_xor(l, o));
    if (grp == 0 && col < G) {
      ml_lds[h * G + col][0] = m;
      ml_lds[h * G + col][1] = l;
    }
    m = -INFINITY;
    l = 0.f;
  };
  auto compute = [&](int i, bf16x8 (&aop)[4][kSD / 32]) {
    const int h = item_head(i), t0 = item_t0(i);
    const bf16 *qh = qs_hi + (h * G + min(col, G - 1)) * kSD + grp * 8;
    const bf16 *ql = qs_lo + (h * G + min(col, G - 1)) * kSD + grp * 8;
    const bool qok = col < G;
    f32x4 z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kSD / 32; ++ks) {
      const bf16x8 bh = qok ? *reinterpret_cast<const bf16x8 *>(qh + ks * 32) : bf16x8{};
      const bf16x8 bl = qok ? *reinterpret_cast<const bf16x8 *>(ql + ks * 32) : bf16x8{};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        z[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[j][ks], bh, z[j], 0, 0, 0);
        z[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[j][ks], bl, z[j], 0, 0, 0);
      }
    }
    // lane (col < G, grp) holds tokens t0 + 16j + 4*grp + r of query head col
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = t0 + 16 * j + 4 * grp + r;
        if (tok >= S) z[j][r] = -INFINITY;
        mx = fmaxf(mx, z[j][r]);
      }
    if (col < G) {
      float *zrow = zs + (h * G + col) * kZStr + (t0 - s0) + 4 * grp;
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4 *>(zrow + 16 * j) = z[j];
      const float mn = fmaxf(m, mx);
      if (mn != -INFINITY) {
        float acc = l * __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc += __builtin_amdgcn_exp2f(z[j][r] - mn);
        l = acc;
        m = mn;
      }
    }
    if (i % n_groups == n_groups - 1) flush(h);
  };

  // three groups in flight: loads of items i+1 and i+2 overlap item i
  // (unconditional loads, clamped to the last item: exact wait counts)
  if (n_items > 0) {
    load(0, abuf[0]);
    load(min(1, n_items - 1), abuf[1]);
  }
  int i = 0;
  for (; i + 2 < n_items; i += 3) {
    load(i + 2, abuf[2]);
    compute(i, abuf[0]);
    load(min(i + 3, n_items - 1), abuf[0]);
    compute(i + 1, abuf[1]);
    load(min(i + 4, n_items - 1), abuf[1]);
    compute(i + 2, abuf[2]);
  }
  if (i < n_items) compute(i, abuf[0]);
  if (i + 1 < n_items) compute(i + 1, abuf[1]);

  // z and (max, sum) of the chunk to global memory: 16-byte stores,
  // consecutive threads on consecutive tokens of one query head
  __syncthreads();
  for (int hq = tid; hq < a.Hq; hq += kThreads) {
    float *pp = w.part + (((int64_t)b * a.Hq + hq) * w.nch_scan + c) * 2;
    pp[0] = ml_lds[hq][0];
    pp[1] = ml_lds[hq][1];
  }
  {
    const int n4 = (int)cdiv(s_end - s0, 4);
    for (int e = tid; e < a.Hq * n4; e += kThreads) {
      const int hq = e / n4, q4 = e - hq * n4;
      const int tok = s0 + 4 * q4;
      const f32x4 v = *reinterpret_cast<const f32x4 *>(zs + hq * kZStr + 4 * q4);
      float *zp = w.z + ((int64_t)b * a.Hq + hq) * w.zs + tok;
      if (tok + 3 < S) {
        *reinterpret_cast<f32x4 *>(zp) = v;
      } else {
        for (int r = 0; r < 4; ++r)
          if (tok + r < S) zp[r] = v[r];
      }
    }
  }

}

// (max, 1 / sum) of each query head of KV head h's group: merge of the
// scan's chunk partials, wave g for head g, chunks cc = lane, lane + 64, ...,
// then a fixed butterfly (the same result in every block that asks).
// Visible to the block after a barrier.
__device__ inline void group_stats(const SelectArgs &a, const SelPtrs &w, int b, int h, int S,
                                   float *st_m, float *st_il) {
  const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63;
  const int nch = (int)cdiv(S, kTS);
  for (int g = wv; g < a.G; g += kThreads / 64) {
    const float *pp = w.part + ((int64_t)b * a.Hq + h * a.G + g) * w.nch_scan * 2;
    float M = -INFINITY, L = 0.f;
    for (int c0 = ln; c0 < nch; c0 += 64 * 8) {  // 8 loads in flight, merged in order
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int cc = c0 + 64 * u;
        v[u] = cc < nch ? *reinterpret_cast<const float2 *>(pp + cc * 2) : float2{-INFINITY, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + 64 * u < nch) merge_ml(M, L, v[u].x, v[u].y);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) merge_ml(M, L, __shfl_xor(M, o), __shfl_xor(L, o));
    if (ln == 0) {
      st_m[g] = M;
      st_il[g] = 1.f / L;
    }
  }
}

// ------------------------------------------------------------------ score
// Block = (chunk of kScoreTok tokens, KV head, row); 4 consecutive tokens per
// thread.
__global__ __launch_bounds__(kThreads) void sel_score_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0) return;
  constexpr int per = kScoreTok / kThreads;
  if (c * kScoreTok >= S) return;
  __shared__ float st_m[8], st_il[8];
  group_stats(a, w, b, h, S, st_m, st_il);
  __shared__ uint32_t hist[kBins];
  for (int e = threadIdx.x; e < kBins; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int s = c * kScoreTok + threadIdx.x * per;
  const bool full = s + per <= S;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // z of every query head of the group loaded first (G <= 8), then summed
  // over the heads in order
  f32x4 zg[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    zg[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (g < a.G) {
      const float *zp = w.z + ((int64_t)b * a.Hq + h * a.G + g) * w.zs + s;
      if (full) {
        zg[g] = *reinterpret_cast<const f32x4 *>(zp);
      } else {
#pragma unroll
        for (int r = 0; r < per; ++r) zg[g][r] = (s + r < S) ? zp[r] : 0.f;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (g < a.G) {
      const float M = st_m[g];
      const float inv_l = st_il[g];
#pragma unroll
      for (int r = 0; r < per; ++r) acc[r] += __builtin_amdgcn_exp2f(zg[g][r] - M) * inv_l;
    }
  }
  float *op = w.scores + ((int64_t)b * a.Hkv + h) * a.s_max + s;
  if (full && ((uintptr_t)op & 15) == 0) {
    *reinterpret_cast<f32x4 *>(op) = acc;
  } else {
#pragma unroll
    for (int r = 0; r < per; ++r)
      if (s + r < S) op[r] = acc[r];
  }
  {  // first radix digit (bits 31..21) of the scores just written
#pragma unroll
    for (int r = 0; r < per; ++r) hist_add(hist, __float_as_uint(acc[r]) >> 21, s + r < S);
    __syncthreads();
    uint32_t *gh = w.hist + ((size_t)b * a.Hkv + h) * 3 * kBins;
    for (int e = threadIdx.x; e < kBins; e += kThreads)
      if (hist[e]) atomicAdd(&gh[e], hist[e]);
  }
}

// ----------------------------------------------------------------- output
// HERALD Sec. IV-B4 keeps, beside the scores, the running output o_g of the
// representative query for every query head and hands it back at once (the
// next layer's FFN waits for it).  Here: o[g] = sum_s p[g, s] V[s, h] with
// p[g, s] = exp2(z[g, s] - m_g) / l_g, the weights the scores sum.  Block =
// (chunk of kOTok tokens, KV head, row) in rounds of 256 tokens: the round's
// weights go to LDS (thread t forms token t's), then thread (token group tg,
// dims 8 dc .. 8 dc + 7) reads 16 value rows (16 lanes read one 256-byte
// row) and accumulates G x 8 sums; the 16 token groups are added by two
// lane exchanges and a fixed-order sum over the 4 waves.
__global__ __launch_bounds__(kThreads) void sel_out_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0 || c * kOTok >= S) return;
  __shared__ float st_m[8], st_il[8];
  group_stats(a, w, b, h, S, st_m, st_il);
  __syncthreads();
  __shared__ float ps[8][kThreads];     // weights of the round's tokens
  __shared__ float red[4][8][kSD];      // per-wave sums
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int dc = lane & 15;
  const int tg = wv * 4 + (lane >> 4);  // tokens tg + 16 i of a round
  float acc[8][8];
#pragma unroll
  for (int g = 0; g < 8; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  const bf16 *vb = a.v + (int64_t)b * a.vs[0] + (int64_t)h * a.vs[2] + dc * 8;
  const int s_end = min(S, (c + 1) * kOTok);
  for (int s0 = c * kOTok; s0 < s_end; s0 += kThreads) {
    {
      const int s = s0 + t;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if (g < a.G) {
          float p = 0.f;
          if (s < s_end)
            p = __builtin_amdgcn_exp2f(w.z[((int64_t)b * a.Hq + h * a.G + g) * w.zs + s] - st_m[g]) * st_il[g];
          ps[g][t] = p;
        }
      }
    }
    __syncthreads();
    bf16x8 vv[16];   // rows past the prefix read its last row (weight 0)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = min(s0 + tg + 16 * i, S - 1);
      vv[i] = *reinterpret_cast<const bf16x8 *>(vb + (int64_t)s * a.vs[1]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = tg + 16 * i;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if (g < a.G) {
          const float p = ps[g][j];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = __builtin_fmaf(p, (float)vv[i][e], acc[g][e]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (g < a.G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[g][e];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        if (lane < 16) red[wv][g][dc * 8 + e] = x;
      }
    }
  }
  __syncthreads();
  float *op = w.opart + (((int64_t)b * a.Hkv + h) * w.nch_o + c) * (a.G * kSD);
  for (int o = t; o < a.G * kSD; o += kThreads) {
    const int g = o / kSD, dd = o - g * kSD;
    op[o] = ((red[0][g][dd] + red[1][g][dd]) + red[2][g][dd]) + red[3][g][dd];
  }
}

// Block = (query head, row), 4 threads per dimension: thread (j, dd) adds
// the partials of chunks j, j + 4, ... in order, then the four sums are
// added in a fixed order; rows without a prefix or a budget get zeros.
__global__ __launch_bounds__(4 * kSD) void sel_out_merge_kernel(SelectArgs a, SelPtrs w) {
  const int hq = blockIdx.x, b = blockIdx.y;
  const int dd = threadIdx.x & (kSD - 1), j = threadIdx.x / kSD;
  int S, kb;
  row_sizes(a, b, S, kb);
  bf16 *o = a.o_rep + ((int64_t)b * a.Hq + hq) * kSD + dd;
  if (S == 0 || kb == 0) {
    if (j == 0) *o = (bf16)0.f;
    return;
  }
  const int h = hq / a.G, g = hq - h * a.G;
  const int nch = (int)cdiv(S, kOTok);
  const int64_t cstr = (int64_t)a.G * kSD;
  const float *pp = w.opart + ((int64_t)b * a.Hkv + h) * w.nch_o * cstr + g * kSD + dd;
  float acc = 0.f;
  for (int c0 = j; c0 < nch; c0 += 4 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c0 + 4 * u < nch ? pp[(c0 + 4 * u) * cstr] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + 4 * u < nch) acc += v[u];
  }
  __shared__ float part[4][kSD];
  part[j][dd] = acc;
  __syncthreads();
  if (j == 0) *o = (bf16)(((part[0][dd] + part[1][dd]) + part[2][dd]) + part[3][dd]);
}

// ---------------------------------------------------------------- top-k
// Digit D with count(digit > D) < krem <= count(digit >= D) over nb bins;
// returns D and the rank left inside it.  Called by every thread of a block
// of 256 or 1024 threads.
__device__ inline void find_digit(const uint32_t *cnt_of, int nb, uint32_t krem, int *sh,
                                  uint32_t &D, uint32_t &rem) {
  (void)sh;
  // wave 0 alone: lane l sums bins nb-1-l*per .. down (per = nb/64, all its
  // loads in flight), one wave-level inclusive scan from the highest bins,
  // and the one lane whose range holds the krem-th count walks its bins
  __shared__ uint32_t sd[2];
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    if (lane == 0) {
      sd[0] = 0;
      sd[1] = krem;
    }
    const int per = nb >> 6;   // 32 or 16 bins per lane, descending
    const int hi_bin = nb - 1 - lane * per;
    uint32_t cnt[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) cnt[e] = e < per ? cnt_of[hi_bin - e] : 0u;
    uint32_t tsum = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) tsum += cnt[e];
    uint32_t x = tsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    const uint32_t before = x - tsum;
    if (before < krem && krem <= x) {
      uint32_t cum = before;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        if (e < per && cum + cnt[e] >= krem) {
          sd[0] = (uint32_t)(hi_bin - e);
          sd[1] = krem - cum;
          break;
        }
        cum += cnt[e];
      }
    }
  }
  __syncthreads();
  D = sd[0];
  rem = sd[1];
  __syncthreads();
}

// Radix select + ordered compaction over keys[0, S) (LDS or global memory).
// Scores cached in LDS with one pad word per 16 (no bank conflicts when a
// thread walks 16 consecutive scores, or when lanes walk consecutive ones).
__device__ inline int cpos(int s) { return s + (s >> 4); }

__device__ inline void topk_body(const uint32_t *keys, int S, int keff, int32_t *out, uint32_t *hist,
                                 int *sh, const uint32_t *hist0) {
  uint32_t prefix = 0, krem = (uint32_t)keff;
  int total_eq = 0;  // scores equal to the threshold (the last digit's count)
  {  // digit 0: the histogram the score pass built while writing the scores
    uint32_t D;
    find_digit(hist0, kBins, krem, sh, D, krem);
    prefix = D << 21;
  }
#pragma unroll 1
  for (int pass = 1; pass < 3; ++pass) {
    const int shift = pass == 1 ? 10 : 0;
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    const int hi_shift = shift + (pass == 2 ? 10 : 11);  // bits above this digit
    for (int e = threadIdx.x; e < kBins; e += kTopkThreads) hist[e] = 0;
    __syncthreads();
    // kRankU keys per thread per round: their LDS reads are issued together,
    // then the histogram updates (the reads' latencies overlap)
    for (int s0 = 0; s0 < S; s0 += kTopkThreads * kRankU) {
      uint32_t kk[kRankU];
#pragma unroll
      for (int u = 0; u < kRankU; ++u) {
        const int s = s0 + u * kTopkThreads + threadIdx.x;
        kk[u] = s < S ? keys[cpos(s)] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kRankU; ++u) {
        const int s = s0 + u * kTopkThreads + threadIdx.x;
        if (s < S && (kk[u] >> hi_shift) == (prefix >> hi_shift)) atomicAdd(&hist[(kk[u] >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    uint32_t D;
    find_digit(hist, pass == 2 ? 1024 : kBins, krem, sh, D, krem);
    prefix |= D << shift;
    if (pass == 2) total_eq = (int)hist[D];
  }
  const uint32_t thr = prefix;
  const int need_eq = (int)krem;

  if (need_eq == total_eq) {
    // every score equal to the threshold is kept (the usual case): the kept
    // set is the scores >= thr, one prefix sum per chunk
    int sel_base = 0;
    for (int c0 = 0; c0 < S; c0 += kTopkThreads * kPerThread) {
      const int sb = c0 + threadIdx.x * kPerThread;
      uint32_t selbits = 0;
      int n_sel = 0;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        const int s = sb + e;
        const bool sel = s < S && keys[cpos(s)] >= thr;
        selbits |= (uint32_t)sel << e;
        n_sel += sel;
      }
      int tot_sel;
      int pos = sel_base + block_excl_scan(n_sel, sh, tot_sel);
#pragma unroll
      for (int e = 0; e < kPerThread; ++e)
        if (selbits & (1u << e)) {
          if (pos < keff) out[pos] = sb + e;
          ++pos;
        }
      sel_base += tot_sel;
    }
    return;
  }

  // ordered compaction: kPerThread consecutive scores per thread per chunk
  int sel_base = 0, eq_base = 0;  // selections / ties before the current chunk
  for (int c0 = 0; c0 < S; c0 += kTopkThreads * kPerThread) {
    const int sb = c0 + threadIdx.x * kPerThread;
    uint32_t kv[kPerThread];
    int n_eq = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int s = sb + e;
      kv[e] = s < S ? keys[cpos(s)] : 0u;
      n_eq += s < S && kv[e] == thr;
    }
    int tot_eq;
    const int eq_rank0 = eq_base + block_excl_scan(n_eq, sh, tot_eq);
    int n_sel = 0, er = eq_rank0;
    uint32_t selbits = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int s = sb + e;
      bool sel = false;
      if (s < S) {
        if (kv[e] > thr) {
          sel = true;
        } else if (kv[e] == thr) {
          sel = er < need_eq;
          ++er;
        }
      }
      selbits |= (uint32_t)sel << e;
      n_sel += sel;
    }
    int tot_sel;
    int pos = sel_base + block_excl_scan(n_sel, sh, tot_sel);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (selbits & (1u << e)) {
        if (pos < keff) out[pos] = sb + e;
        ++pos;
      }
    sel_base += tot_sel;
    eq_base += tot_eq;
  }
}

__global__ __launch_bounds__(kTopkThreads) void sel_topk_kernel(SelectArgs a, SelPtrs w) {
  const int p = blockIdx.x;
  const int b = p / a.Hkv;
  int S, kb;
  row_sizes(a, b, S, kb);
  const int keff = min(S, kb);
  int32_t *out = a.idx_out + (size_t)p * a.k_max;
  for (int j = keff + threadIdx.x; j < a.k_max; j += kTopkThreads) out[j] = -1;
  if (keff == 0) return;
  if (keff == S) {  // the whole prefix is selected
    for (int j = threadIdx.x; j < S; j += kTopkThreads) out[j] = j;
    return;
  }
  __shared__ uint32_t hist[kBins];
  __shared__ int sh[16];
  __shared__ uint32_t cache[kLdsKeys + kLdsKeys / 16];
  const uint32_t *keys = reinterpret_cast<const uint32_t *>(w.scores) + (size_t)p * a.s_max;
  // S <= kLdsKeys; 16 loads in flight per thread
  for (int e0 = threadIdx.x; e0 < S; e0 += kTopkThreads * 16) {
    uint32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = e0 + kTopkThreads * u;
      v[u] = e < S ? keys[e] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = e0 + kTopkThreads * u;
      if (e < S) cache[cpos(e)] = v[u];
    }
  }
  __syncthreads();
  topk_body(cache, S, keff, out, hist, sh, w.hist + (size_t)p * 3 * kBins);
}

// ------------------------------------------------------ multi-block ranking
// Rows longer than kLdsKeys: blocks of kCK scores.  Each kernel recomputes
// the digits fixed so far from the global histograms (kernel boundaries
// order the histogram updates; no fences).

// Threshold prefix and remaining rank after `passes` digits.
__device__ inline void known_digits(const SelPtrs &w, int p, uint32_t keff, int passes, int *sh,
                                    uint32_t &prefix, uint32_t &krem) {
  prefix = 0;
  krem = keff;
  for (int d = 0; d < passes; ++d) {
    uint32_t D;
    find_digit(w.hist + ((size_t)p * 3 + d) * kBins, d == 2 ? 1024 : kBins, krem, sh, D, krem);
    prefix |= D << (d == 0 ? 21 : (d == 1 ? 10 : 0));
  }
}

__device__ inline bool rank_sizes(const SelectArgs &a, int p, int c, int &S, int &keff) {
  int kb;
  row_sizes(a, p / a.Hkv, S, kb);
  keff = min(S, kb);
  return keff > 0 && keff < S && c * kCK < S;
}

// Histogram of digit PASS + 1 (bits 20..10, then 9..0) over one block of
// scores whose higher digits match the threshold's.
template <int PASS>
__global__ __launch_bounds__(kThreads) void sel_hist_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, p = blockIdx.y;
  int S, keff;
  if (!rank_sizes(a, p, c, S, keff)) return;
  __shared__ uint32_t hist[kBins];
  __shared__ int sh[16];
  uint32_t prefix, krem;
  known_digits(w, p, (uint32_t)keff, PASS, sh, prefix, krem);
  for (int e = threadIdx.x; e < kBins; e += kThreads) hist[e] = 0;
  __syncthreads();
  constexpr int shift = PASS == 1 ? 10 : 0;
  constexpr uint32_t dmask = PASS == 1 ? 2047u : 1023u;
  constexpr int hi_shift = PASS == 1 ? 21 : 10;
  const uint32_t *keys = reinterpret_cast<const uint32_t *>(w.scores) + (size_t)p * a.s_max;
  uint32_t kv[kCK / kThreads];  // all loads in flight before the histogram updates
#pragma unroll
  for (int e = 0; e < kCK / kThreads; ++e) {
    const int s = c * kCK + e * kThreads + threadIdx.x;
    kv[e] = s < S ? keys[s] : 0u;
  }
#pragma unroll
  for (int e = 0; e < kCK / kThreads; ++e) {
    const int s = c * kCK + e * kThreads + threadIdx.x;
    const uint32_t key = kv[e];
    hist_add(hist, (key >> shift) & dmask, s < S && (key >> hi_shift) == (prefix >> hi_shift));
  }
  __syncthreads();
  uint32_t *gh = w.hist + ((size_t)p * 3 + PASS) * kBins;
  for (int e = threadIdx.x; e < kBins; e += kThreads)
    if (hist[e]) atomicAdd(&gh[e], hist[e]);
}

// Per block: scores above the threshold and equal to it.
__global__ __launch_bounds__(kThreads) void sel_count_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, p = blockIdx.y;
  int S, keff;
  if (!rank_sizes(a, p, c, S, keff)) return;
  __shared__ int sh[16];
  uint32_t thr, krem;
  known_digits(w, p, (uint32_t)keff, 3, sh, thr, krem);
  const uint32_t *keys = reinterpret_cast<const uint32_t *>(w.scores) + (size_t)p * a.s_max;
  int gt = 0, eq = 0;
  uint32_t kv[kCK / kThreads];
#pragma unroll
  for (int e = 0; e < kCK / kThreads; ++e) {
    const int s = c * kCK + e * kThreads + threadIdx.x;
    kv[e] = s < S ? keys[s] : 0u;
  }
#pragma unroll
  for (int e = 0; e < kCK / kThreads; ++e) {
    const int s = c * kCK + e * kThreads + threadIdx.x;
    if (s < S) {
      gt += kv[e] > thr;
      eq += kv[e] == thr;
    }
  }
  int tg, te;
  block_excl_scan(gt, sh, tg);
  block_excl_scan(eq, sh, te);
  if (threadIdx.x == 0) {
    w.ccount[((size_t)p * w.nch_topk + c) * 2 + 0] = (uint32_t)tg;
    w.ccount[((size_t)p * w.nch_topk + c) * 2 + 1] = (uint32_t)te;
  }
}

// Ordered compaction of one block: positions after every earlier block's
// selections; ties by position up to the threshold's remaining rank.  Block 0
// also writes the -1 padding.  Rows whose budget covers the whole prefix
// select every position.
__global__ __launch_bounds__(kThreads) void sel_write_kernel(SelectArgs a, SelPtrs w) {
  const int c = blockIdx.x, p = blockIdx.y;
  int S, kb;
  row_sizes(a, p / a.Hkv, S, kb);
  const int keff = min(S, kb);
  int32_t *out = a.idx_out + (size_t)p * a.k_max;
  if (c == 0)
    for (int j = keff + threadIdx.x; j < a.k_max; j += kThreads) out[j] = -1;
  if (keff == 0 || c * kCK >= S) return;
  if (keff == S) {
    for (int j = c * kCK + threadIdx.x; j < min(S, (c + 1) * kCK); j += kThreads) out[j] = j;
    return;
  }
  __shared__ int sh[16];
  uint32_t thr, krem;
  known_digits(w, p, (uint32_t)keff, 3, sh, thr, krem);
  const int need_eq = (int)krem;
  int gtb = 0, eqb = 0;
  for (int cc = threadIdx.x; cc < c; cc += kThreads) {
    gtb += (int)w.ccount[((size_t)p * w.nch_topk + cc) * 2 + 0];
    eqb += (int)w.ccount[((size_t)p * w.nch_topk + cc) * 2 + 1];
  }
  int gt_before, eq_before;
  block_excl_scan(gtb, sh, gt_before);
  block_excl_scan(eqb, sh, eq_before);
  constexpr int per = kCK / kThreads;  // 16 consecutive scores per thread
  const int s0 = c * kCK + threadIdx.x * per;
  const uint32_t *keys = reinterpret_cast<const uint32_t *>(w.scores) + (size_t)p * a.s_max;
  uint32_t kv[per];
  int n_eq = 0;
#pragma unroll
  for (int e = 0; e < per; ++e) {
    const int s = s0 + e;
    kv[e] = s < S ? keys[s] : 0u;
    n_eq += s < S && kv[e] == thr;
  }
  int tot;
  int er = eq_before + block_excl_scan(n_eq, sh, tot);
  int n_sel = 0;
  uint32_t selbits = 0;
#pragma unroll
  for (int e = 0; e < per; ++e) {
    const int s = s0 + e;
    bool sel = false;
    if (s < S) {
      if (kv[e] > thr) {
        sel = true;
      } else if (kv[e] == thr) {
        sel = er < need_eq;
        ++er;
      }
    }
    selbits |= (uint32_t)sel << e;
    n_sel += sel;
  }
  int pos = gt_before + min(eq_before, need_eq) + block_excl_scan(n_sel, sh, tot);
#pragma unroll
  for (int e = 0; e < per; ++e)
    if (selbits & (1u << e)) {
      if (pos < keff) out[pos] = s0 + e;
      ++pos;
    }
}

// ------------------------------------------------ exact multi-query selection
// Every one of the nq block queries ranks the prefix (HERALD Sec. III-C and
// Sec. IV-A2, the selection phase before the query reduction).  The columns
// of KV head h are the nq*G pairs (query i, group head g), column c = i*G+g,
// at most kMCols.  Two passes over K; no score matrix is stored:
//   stats  per kMTok-token chunk and column, the (max, sum) of the logits in
//          log2 units, from S = K Q^T with the tokens on the M side of
//          v_mfma_f32_16x16x32_bf16 (a lane holds 4 tokens of one column, so
//          the running statistics are lane-local).
//   merge  fixed-order merge of the chunks: mp[c] = m_c + log2(l_c).
//   score  the same dot products with the columns on the M side (a lane
//          holds 4 columns of one token); s_hat[s] = sum_c exp2(z - mp[c]),
//          written once: these are the values the top-k kernels rank.
// The K fragments are loaded straight into registers (a lane reads 16 bytes
// of 4 k-groups of one token: 64 contiguous bytes per token per load); the
// next 64-token group is in flight while the current one is computed.  The
// query columns (raw bf16, scaled after the MFMA in fp32) sit in LDS.
constexpr int kMTok = 1024;     // tokens per block of the two passes
constexpr int kMCols = 128;     // columns (query, group head) per KV head
constexpr int kQStr = kSD + 8;  // LDS row stride of the staged columns (elements)

struct MultiLayout {
  size_t part, mp, scores, hist, ccount, total;
  int nch, nch_topk;
  bool multi;
};

MultiLayout multi_layout(int B, int Hkv, int s_max) {
  MultiLayout L;
  L.nch = (int)cdiv(s_max > 0 ? s_max : 1, kMTok);
  L.nch_topk = (int)cdiv(s_max > 0 ? s_max : 1, kCK);
  L.multi = s_max > kLdsKeys;
  const size_t P = (size_t)B * Hkv;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  L.part = take(P * kMCols * (size_t)L.nch * 2 * 4);
  L.mp = take(P * kMCols * 4);
  L.scores = take(P * (size_t)s_max * 4);
  L.hist = take(P * 3 * kBins * 4);
  L.ccount = L.multi ? take(P * L.nch_topk * 2 * 4) : 0;
  L.total = off;
  return L;
}

struct MultiPtrs {
  float *part, *mp, *scores;
  uint32_t *hist;
  int nch, ncol;
  bool multi;
};

// Query columns of (row b, KV head h) into LDS, zero past ncol up to ncp.
__device__ inline void stage_columns(const SelectArgs &a, int b, int h, int ncol, int ncp, bf16 *qs) {
  for (int e = threadIdx.x; e < ncp * 16; e += blockDim.x) {
    const int c = e >> 4, piece = e & 15;
    bf16x8 v = bf16x8{};
    if (c < ncol) {
      const int i = c / a.G, g = c - i * a.G;
      v = *reinterpret_cast<const bf16x8 *>(a.q + (int64_t)b * a.qs[0] + (int64_t)i * a.qs[1] +
                                            (int64_t)(h * a.G + g) * a.qs[2] + piece * 8);
    }
    *reinterpret_cast<bf16x8 *>(qs + c * kQStr + piece * 8) = v;
  }
}

// K fragments of one 64-token group: kf[tb][ks] holds token
// t0 + 16*tb + (lane & 15), dims 32*ks + 8*(lane >> 4) .. +8.  Tokens past S
// re-read token S-1 (their logits are masked or their scores not written).
__device__ inline void load_group(const bf16 *kbase, int64_t kstride, int t0, int S, bf16x8 (&kf)[4][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int tok = min(t0 + 16 * tb + (lane & 15), S - 1);
    const bf16 *kp = kbase + (int64_t)tok * kstride + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kf[tb][ks] = *reinterpret_cast<const bf16x8 *>(kp + 32 * ks);
  }
}

// Block = (chunk of kMTok tokens, KV head, row), 4 waves; wave w takes the
// 64-token groups w, w+4, w+8, w+12 of the chunk.
__global__ __launch_bounds__(kThreads, 2) void selm_stats_kernel(SelectArgs a, MultiPtrs w) {
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0 || c * kMTok >= S) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncol = w.ncol, ncb = (ncol + 15) >> 4;
  __shared__ __attribute__((aligned(16))) bf16 qs[kMCols * kQStr];
  __shared__ float ml_lds[4][kMCols][2];
  stage_columns(a, b, h, ncol, ncb * 16, qs);
  __syncthreads();

  const int s0 = c * kMTok, s_end = min(s0 + kMTok, S);
  const int ng_all = (int)cdiv(s_end - s0, 64);
  const int ng = ng_all > wave ? (int)cdiv(ng_all - wave, 4) : 0;   // this wave's groups
  const bf16 *kbase = a.k + (int64_t)b * a.ks[0] + (int64_t)h * a.ks[2];
  float m[8], l[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    m[cb] = -INFINITY;
    l[cb] = 0.f;
  }
  auto t0_of = [&](int j) { return s0 + 64 * (wave + 4 * min(j, ng - 1)); };
  auto compute = [&](int j, bf16x8 (&kf)[4][4]) {
    const int t0 = t0_of(j);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      if (cb >= ncb) break;
      bf16x8 qf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[ks] = *reinterpret_cast<const bf16x8 *>(qs + (cb * 16 + (lane & 15)) * kQStr + 32 * ks + 8 * (lane >> 4));
      f32x4 z[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) z[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) z[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tb][ks], qf[ks], z[tb], 0, 0, 0);
      // lane holds tokens t0 + 16*tb + 4*(lane >> 4) + r of column cb*16 + (lane & 15)
      float mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          z[tb][r] *= a.scale2;
          if (t0 + 16 * tb + 4 * (lane >> 4) + r >= S) z[tb][r] = -INFINITY;
          mx = fmaxf(mx, z[tb][r]);
        }
      const float mn = fmaxf(m[cb], mx);
      if (mn != -INFINITY) {
        float acc = l[cb] * __builtin_amdgcn_exp2f(m[cb] - mn);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc += __builtin_amdgcn_exp2f(z[tb][r] - mn);
        l[cb] = acc;
        m[cb] = mn;
      }
    }
  };
  if (ng > 0) {
    bf16x8 ka[4][4], kb2[4][4];
    load_group(kbase, a.ks[1], t0_of(0), S, ka);
    load_group(kbase, a.ks[1], t0_of(1), S, kb2);
    compute(0, ka);
    load_group(kbase, a.ks[1], t0_of(2), S, ka);
    if (1 < ng) compute(1, kb2);
    load_group(kbase, a.ks[1], t0_of(3), S, kb2);
    if (2 < ng) compute(2, ka);
    if (3 < ng) compute(3, kb2);
  }
  // merge the 4 lane groups holding the same column, then the 4 waves
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    if (cb >= ncb) break;
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) merge_ml(m[cb], l[cb], __shfl_xor(m[cb], o), __shfl_xor(l[cb], o));
    if (lane < 16) {
      ml_lds[wave][cb * 16 + lane][0] = m[cb];
      ml_lds[wave][cb * 16 + lane][1] = l[cb];
    }
  }
  __syncthreads();
  for (int col = tid; col < ncol; col += kThreads) {
    float M = -INFINITY, Lsum = 0.f;
    for (int wv = 0; wv < 4; ++wv) merge_ml(M, Lsum, ml_lds[wv][col][0], ml_lds[wv][col][1]);
    float *pp = w.part + ((((int64_t)b * a.Hkv + h) * kMCols + col) * w.nch + c) * 2;
    pp[0] = M;
    pp[1] = Lsum;
  }
}

// Block = (KV head, row), kMCols threads: mp[c] = m_c + log2(l_c) over the
// chunks in order; clears the row's digit histograms for the ranking.
__global__ __launch_bounds__(kMCols) void selm_merge_kernel(SelectArgs a, MultiPtrs w) {
  const int h = blockIdx.x, b = blockIdx.y;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0) return;
  const int nch = (int)cdiv(S, kMTok);
  const int col = threadIdx.x;
  if (col < w.ncol) {
    const float *pp = w.part + (((int64_t)b * a.Hkv + h) * kMCols + col) * w.nch * 2;
    float M = -INFINITY, Lsum = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 8) {  // 8 loads in flight, merged in order
      float2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = c0 + u < nch ? *reinterpret_cast<const float2 *>(pp + (c0 + u) * 2) : float2{-INFINITY, 0.f};
#pragma unroll
      for (int u = 0; u < 8; ++u) merge_ml(M, Lsum, v[u].x, v[u].y);
    }
    w.mp[((int64_t)b * a.Hkv + h) * kMCols + col] = M + __log2f(Lsum);
  }
  {
    uint32_t *hist = w.hist + ((size_t)b * a.Hkv + h) * 3 * kBins;
    for (int e = threadIdx.x; e < 3 * kBins; e += kMCols) hist[e] = 0;
  }
}

// Block = (chunk of kMTok tokens, KV head, row), 4 waves as in the stats pass.
__global__ __launch_bounds__(kThreads, 2) void selm_score_kernel(SelectArgs a, MultiPtrs w) {
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int S, kb;
  row_sizes(a, b, S, kb);
  if (S == 0 || kb == 0 || c * kMTok >= S) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncol = w.ncol, ncb = (ncol + 15) >> 4;
  __shared__ __attribute__((aligned(16))) bf16 qs[kMCols * kQStr];
  __shared__ __attribute__((aligned(16))) float mps[kMCols];
  __shared__ uint32_t hist[kBins];
  stage_columns(a, b, h, ncol, ncb * 16, qs);
  for (int col = tid; col < kMCols; col += kThreads)
    mps[col] = col < ncol ? w.mp[((int64_t)b * a.Hkv + h) * kMCols + col] : INFINITY;
  for (int e = tid; e < kBins; e += kThreads) hist[e] = 0;
  __syncthreads();

  const int s0 = c * kMTok, s_end = min(s0 + kMTok, S);
  const int ng_all = (int)cdiv(s_end - s0, 64);
  const int ng = ng_all > wave ? (int)cdiv(ng_all - wave, 4) : 0;
  const bf16 *kbase = a.k + (int64_t)b * a.ks[0] + (int64_t)h * a.ks[2];
  float *orow = w.scores + ((int64_t)b * a.Hkv + h) * a.s_max;
  auto t0_of = [&](int j) { return s0 + 64 * (wave + 4 * min(j, ng - 1)); };
  auto compute = [&](int j, bf16x8 (&kf)[4][4]) {
    const int t0 = t0_of(j);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      if (cb >= ncb) break;
      bf16x8 qf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[ks] = *reinterpret_cast<const bf16x8 *>(qs + (cb * 16 + (lane & 15)) * kQStr + 32 * ks + 8 * (lane >> 4));
      // columns cb*16 + 4*(lane >> 4) + r of the lane
      const f32x4 mp = *reinterpret_cast<const f32x4 *>(mps + cb * 16 + 4 * (lane >> 4));
      f32x4 z[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) z[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) z[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], kf[tb][ks], z[tb], 0, 0, 0);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[tb] += __builtin_amdgcn_exp2f(__builtin_fmaf(z[tb][r], a.scale2, -mp[r]));
    }
    // sum over the 4 lane groups (the other columns), fixed butterfly
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      acc[tb] += __shfl_xor(acc[tb], 16);
      acc[tb] += __shfl_xor(acc[tb], 32);
    }
    // lane L writes token t0 + L: token block L >> 4, token L & 15 of it
    const int grp = lane >> 4;
    const float v = grp == 0 ? acc[0] : (grp == 1 ? acc[1] : (grp == 2 ? acc[2] : acc[3]));
    const int tok = t0 + lane;
    if (tok < S) orow[tok] = v;
    hist_add(hist, __float_as_uint(v) >> 21, tok < S);
  };
  if (ng > 0) {
    bf16x8 ka[4][4], kb2[4][4];
    load_group(kbase, a.ks[1], t0_of(0), S, ka);
    load_group(kbase, a.ks[1], t0_of(1), S, kb2);
    compute(0, ka);
    load_group(kbase, a.ks[1], t0_of(2), S, ka);
    if (1 < ng) compute(1, kb2);
    load_group(kbase, a.ks[1], t0_of(3), S, kb2);
    if (2 < ng) compute(2, ka);
    if (3 < ng) compute(3, kb2);
  }
  {  // first radix digit of the scores just written
    __syncthreads();
    uint32_t *gh = w.hist + ((size_t)b * a.Hkv + h) * 3 * kBins;
    for (int e = tid; e < kBins; e += kThreads)
      if (hist[e]) atomicAdd(&gh[e], hist[e]);
  }
}

// Top-k of the scores in w.scores (one LDS block per row, or the
// multi-block ranking for rows longer than kLdsKeys).
hipError_t launch_rank(const SelectArgs &a, const SelPtrs &w, hipStream_t s) {
  if (!w.multi) {
    hipLaunchKernelGGL(sel_topk_kernel, dim3(a.B * a.Hkv), dim3(kTopkThreads), 0, s, a, w);
    return hipGetLastError();
  }
  const dim3 tg(w.nch_topk, a.B * a.Hkv);
  hipLaunchKernelGGL(sel_hist_kernel<1>, tg, dim3(kThreads), 0, s, a, w);
  hipLaunchKernelGGL(sel_hist_kernel<2>, tg, dim3(kThreads), 0, s, a, w);
  hipLaunchKernelGGL(sel_count_kernel, tg, dim3(kThreads), 0, s, a, w);
  hipLaunchKernelGGL(sel_write_kernel, tg, dim3(kThreads), 0, s, a, w);
  return hipGetLastError();
}

}  // namespace

size_t select_workspace(int B, int Hq, int Hkv, int d, int s_max, int k_max, bool with_out) {
  (void)k_max;
  return sel_layout(B, Hq, Hkv, d, s_max, with_out).total;
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  const bool with_out = a.o_rep != nullptr;
  const SelLayout L = sel_layout(a.B, a.Hq, a.Hkv, a.d, a.s_max, with_out);
  SelPtrs w;
  w.qhi = reinterpret_cast<bf16 *>(a.ws + L.qhi);
  w.qlo = reinterpret_cast<bf16 *>(a.ws + L.qlo);
  w.z = reinterpret_cast<float *>(a.ws + L.z);
  w.part = reinterpret_cast<float *>(a.ws + L.part);
  w.scores = a.score_out ? a.score_out : reinterpret_cast<float *>(a.ws + L.scores);
  w.nch_scan = L.nch_scan;
  w.zs = L.zs;
  w.nch_topk = L.nch_topk;
  w.multi = L.multi;
  w.hist = reinterpret_cast<uint32_t *>(a.ws + L.hist);
  w.ccount = reinterpret_cast<uint32_t *>(a.ws + L.ccount);
  w.opart = reinterpret_cast<float *>(a.ws + L.opart);
  w.nch_o = L.nch_o;
  hipError_t e;
  if (a.k_max == 0) {   // no row selects: only the output rows (zeros)
    if (with_out) hipLaunchKernelGGL(sel_out_merge_kernel, dim3(a.Hq, a.B), dim3(4 * kSD), 0, s, a, w);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(sel_prep_kernel, dim3(a.Hq, a.B), dim3(kThreads), 0, s, a, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t scan_lds = (size_t)a.Hq * (2 * kSD * sizeof(bf16) + kZStr * sizeof(float));
  hipLaunchKernelGGL(sel_scan_kernel, dim3(L.nch_scan, a.B), dim3(kThreads), scan_lds, s, a, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.s_max > 0)   // (no prefix anywhere: the rank pass writes the -1 rows)
    hipLaunchKernelGGL(sel_score_kernel, dim3((unsigned)cdiv(a.s_max, kScoreTok), a.Hkv, a.B),
                       dim3(kThreads), 0, s, a, w);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (with_out) {
    if (a.s_max > 0)
      hipLaunchKernelGGL(sel_out_kernel, dim3((unsigned)L.nch_o, a.Hkv, a.B), dim3(kThreads), 0, s, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(sel_out_merge_kernel, dim3(a.Hq, a.B), dim3(4 * kSD), 0, s, a, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return launch_rank(a, w, s);
}

size_t select_multi_workspace(int B, int Hkv, int s_max) { return multi_layout(B, Hkv, s_max).total; }

hipError_t launch_select_multi(const SelectArgs &a, hipStream_t s) {
  const MultiLayout L = multi_layout(a.B, a.Hkv, a.s_max);
  MultiPtrs m;
  m.part = reinterpret_cast<float *>(a.ws + L.part);
  m.mp = reinterpret_cast<float *>(a.ws + L.mp);
  m.scores = a.score_out ? a.score_out : reinterpret_cast<float *>(a.ws + L.scores);
  m.hist = reinterpret_cast<uint32_t *>(a.ws + L.hist);
  m.nch = L.nch;
  m.ncol = a.nq * a.G;
  m.multi = L.multi;
  SelPtrs w{};
  w.scores = m.scores;
  w.hist = m.hist;
  w.ccount = reinterpret_cast<uint32_t *>(a.ws + L.ccount);
  w.nch_topk = L.nch_topk;
  w.multi = L.multi;
  const dim3 grid(L.nch, a.Hkv, a.B);
  hipError_t e;
  hipLaunchKernelGGL(selm_stats_kernel, grid, dim3(kThreads), 0, s, a, m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(selm_merge_kernel, dim3(a.Hkv, a.B), dim3(kMCols), 0, s, a, m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(selm_score_kernel, grid, dim3(kThreads), 0, s, a, m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_rank(a, w, s);
}

}  // namespace bd

