// Block-diffusion attention: GQA, per-row prefix length, W-shaped window mask
// (FlowBlock review Eq. (6)); HERALD's denoising attention over a pool when
// the prefix is a gathered pool.
//
// MFMA path (bf16, d = 128).  Work unit = (row, KV head h, tile of 32 window
// queries, key chunk).  A 64-lane wave owns one query head of the GQA group,
// so the G waves of a block share every K/V tile staged in LDS.  The wave
// computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on M, queries on
// N): every lane then holds one query's scores, so the online softmax
// (FlashAttention running max / sum) is lane-local apart from one exchange
// with lane l^32.  O^T += V^T P^T reuses the S^T accumulator layout as the B
// operand directly; V is staged transposed in LDS with the key order inside
// each 16-key group permuted to match that layout.
//
// All prefix keys are visible to every query, so the only masked tiles are
// the ragged prefix end and the window part; keys at or past the prefix
// length are never loaded (zero-filled in LDS), which keeps NaN sentinels in
// unused cache rows out of the arithmetic.
//
// Split-KV: when there are too few units to fill the 256 CUs, the prefix is
// cut into chunks; each chunk writes unnormalised partial O with its running
// (max, sum), and a combine kernel merges the chunks in a fixed order.
#include "bd_common.h"

namespace bd {

namespace {

// ----------------------------------------------------------------- MFMA path
constexpr int kD = 128;          // head dim of the MFMA path
constexpr int kTileK = 64;       // keys per staged tile
constexpr int kQT = 32;          // queries per tile (MFMA N)
constexpr int kKStr = kD + 8;    // LDS row stride of K (elements): 272 B
constexpr int kVStr = kTileK + 8;  // LDS row stride of V^T (elements): 144 B

__device__ inline bf16x8 ld_bf16x8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// LDS slot of key k16 (0..15) inside a 16-key group of V^T: bits 2 and 3
// swapped, so that lane half hh reads keys {hh*4 + 0..3, 8 + hh*4 + 0..3},
// the keys its S^T accumulator registers hold.
__device__ inline int vt_slot(int k16) {
  return (k16 & 3) | ((k16 & 4) << 1) | ((k16 & 8) >> 1);
}

template <int G>
__global__ __launch_bounds__(64 * G) void attn_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[kTileK * kKStr];
  __shared__ __attribute__((aligned(16))) bf16 Vt[kD * kVStr];

  constexpr int NT = 64 * G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;     // lane half
  const int ln = lane & 31;     // query column / M row inside a 32x32 tile

  // ---- decode the unit (XCD-aware: the units of one (row, KV head) group
  // are dispatched to the same XCD so its K/V stay in that XCD's L2)
  const int per_group = a.nqt * a.n_split;
  const int n_groups = a.n_rows * a.Hkv;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int kk = bid >> 3;
  const int group = xcd + 8 * (kk / per_group);
  if (group >= n_groups) return;
  const int mem = kk % per_group;
  const int u = mem / a.n_split;
  const int c = mem - u * a.n_split;
  const int rl = group / a.Hkv;
  const int h = group - rl * a.Hkv;
  const int b = a.row_ids ? a.row_ids[rl] : rl;
  if (b < 0 || b >= a.B) return;
  const int P = clampi(a.p_len[b], 0, min(a.p_max, a.p_cap));
  const int nc = P > 0 ? (int)cdiv(P, a.chunk) : 1;
  if (c >= nc) return;
  const int kbeg = c * a.chunk;
  const int kend = min(P, kbeg + a.chunk);
  const bool with_window = (c == nc - 1);
  const int i0 = u * kQT;
  const int ilast = min(i0 + kQT, a.q) - 1;
  const int win_len = window_limit(ilast, a.bl, a.q);
  const int hq = h * G + wave;
  const int qi = i0 + ln;              // this lane's query
  const bool q_ok = qi < a.q;
  const int lim_i = window_limit(q_ok ? qi : ilast, a.bl, a.q);

  // ---- Q operand (B of S^T = K Q^T): lane holds Q[qi][ks*16 + hh*8 .. +8]
  bf16x8 qop[kD / 16];
  {
    const bf16 *qp = reinterpret_cast<const bf16 *>(a.Q) + (int64_t)b * a.qs[0] +
                     (int64_t)qi * a.qs[1] + (int64_t)hq * a.qs[2] + hh * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      if (q_ok)
        qop[ks] = ld_bf16x8(qp + ks * 16);
      else
        qop[ks] = bf16x8{};
    }
  }

  f32x16 acc_o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) acc_o[dt] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled scores (log2 units)
  float l_run = 0.f;        // running sum of exp2(score - m_run)

  const bf16 *pkb = reinterpret_cast<const bf16 *>(a.pk) + (int64_t)b * a.ps[0] + (int64_t)h * a.ps[2];
  const bf16 *pvb = reinterpret_cast<const bf16 *>(a.pv) + (int64_t)b * a.ps[0] + (int64_t)h * a.ps[2];
  const bf16 *wkb = reinterpret_cast<const bf16 *>(a.wk) + (int64_t)b * a.ws[0] + (int64_t)h * a.ws[2];
  const bf16 *wvb = reinterpret_cast<const bf16 *>(a.wv) + (int64_t)b * a.ws[0] + (int64_t)h * a.ws[2];

  const int n_pref_tiles = (kend > kbeg) ? (int)cdiv(kend - kbeg, kTileK) : 0;
  const int n_win_tiles = with_window ? (int)cdiv(win_len, kTileK) : 0;
  const int n_tiles = n_pref_tiles + n_win_tiles;

  for (int tile = 0; tile < n_tiles; ++tile) {
    const bool win = tile >= n_pref_tiles;
    const int base = win ? (tile - n_pref_tiles) * kTileK : kbeg + tile * kTileK;
    const int limit = win ? win_len : kend;
    const bf16 *kb = win ? wkb : pkb;
    const bf16 *vb = win ? wvb : pvb;
    const int64_t sp = win ? a.ws[1] : a.ps[1];

    __syncthreads();  // previous tile fully consumed
    // ---- stage K [64 keys][128 d] row-major, 16 lanes per key row
    for (int piece = tid; piece < kTileK * 16; piece += NT) {
      const int key = piece >> 4;
      const int ch = piece & 15;
      const int gk = base + key;
      bf16x8 v = bf16x8{};
      if (gk < limit) v = ld_bf16x8(kb + (int64_t)gk * sp + ch * 8);
      *reinterpret_cast<bf16x8 *>(&Ks[key * kKStr + ch * 8]) = v;
    }
    // ---- stage V transposed: V^T[d][slot(key)], 4 keys x 8 d per item
    for (int item = tid; item < (kTileK / 4) * (kD / 8); item += NT) {
      const int db = item & 15;
      const int kb4 = item >> 4;  // keys 4*kb4 .. 4*kb4+3
      bf16x8 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gk = base + 4 * kb4 + j;
        v[j] = (gk < limit) ? ld_bf16x8(vb + (int64_t)gk * sp + db * 8) : bf16x8{};
      }
      const int slot = (kb4 >> 2) * 16 + vt_slot((kb4 & 3) * 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 w = {v[0][e], v[1][e], v[2][e], v[3][e]};
        *reinterpret_cast<bf16x4 *>(&Vt[(db * 8 + e) * kVStr + slot]) = w;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for two 32-key sub-tiles
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8 kop = ld_bf16x8(&Ks[(kt * 32 + ln) * kKStr + ks * 16 + hh * 8]);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], s[kt], 0, 0, 0);
      }
    }

    // ---- mask, scale, online softmax (lane = query column)
    const int vlim = win ? lim_i : limit;
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = base + kt * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
        const float v = (key < vlim) ? s[kt][r] * a.scale2 : -INFINITY;
        s[kt][r] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kt][r] - m_use);
        s[kt][r] = p;
        rs += p;
      }
    }
    rs += xor32(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[dt][r] *= alpha;

    // ---- P^T operands: registers 8k..8k+7 of s[kt] -> keys of k-step (kt, k)
    bf16x8 pop[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pop[kt][k2][e] = (bf16)s[kt][8 * k2 + e];

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const bf16x8 vop =
              ld_bf16x8(&Vt[(dt * 32 + ln) * kVStr + kt * 32 + k2 * 16 + hh * 8]);
          acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[kt][k2], acc_o[dt], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue
  if (!q_ok) return;
  if (nc == 1) {
    const float inv = 1.f / l_run;
    bf16 *op = reinterpret_cast<bf16 *>(a.out) + (int64_t)b * a.os[0] + (int64_t)qi * a.os[1] +
               (int64_t)hq * a.os[2];
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc_o[dt][rq * 4 + e] * inv);
        *reinterpret_cast<bf16x4 *>(op + dt * 32 + rq * 8 + hh * 4) = w;
      }
    }
    if (a.lse && hh == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.q + qi] = (m_run + __log2f(l_run)) * kLn2;
  } else {
    const int64_t unit = (int64_t)group * a.nqt + u;
    const int64_t prow = ((unit * a.n_split + c) * G + wave) * kQT + ln;
    float *po = a.part_o + prow * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 w = {acc_o[dt][rq * 4 + 0], acc_o[dt][rq * 4 + 1], acc_o[dt][rq * 4 + 2],
                   acc_o[dt][rq * 4 + 3]};
        *reinterpret_cast<f32x4 *>(po + dt * 32 + rq * 8 + hh * 4) = w;
      }
    if (hh == 0) {
      a.part_ml[prow * 2 + 0] = m_run;
      a.part_ml[prow * 2 + 1] = l_run;
    }
  }
}

// Merge split-KV partials of one unit (row, KV head, query tile): fixed chunk
// order, so the result does not depend on scheduling.
template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, int D) {
  const int unit = blockIdx.x;
  const int group = unit / a.nqt;
  const int u = unit - group * a.nqt;
  const int rl = group / a.Hkv;
  const int h = group - rl * a.Hkv;
  const int b = a.row_ids ? a.row_ids[rl] : rl;
  if (b < 0 || b >= a.B) return;
  const int P = clampi(a.p_len[b], 0, min(a.p_max, a.p_cap));
  const int nc = P > 0 ? (int)cdiv(P, a.chunk) : 1;
  if (nc == 1) return;  // written directly by the attention kernel
  const int rows = a.G * kQT;
  for (int item = threadIdx.x; item < rows * (D / 4); item += blockDim.x) {
    const int row = item / (D / 4);
    const int d4 = item - row * (D / 4);
    const int g = row / kQT;
    const int il = row - g * kQT;
    const int qi = u * kQT + il;
    if (qi >= a.q) continue;
    float M = -INFINITY;
    for (int cc = 0; cc < nc; ++cc) {
      const int64_t prow = (((int64_t)unit * a.n_split + cc) * a.G + g) * kQT + il;
      M = fmaxf(M, a.part_ml[prow * 2]);
    }
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int cc = 0; cc < nc; ++cc) {
      const int64_t prow = (((int64_t)unit * a.n_split + cc) * a.G + g) * kQT + il;
      const float w = __builtin_amdgcn_exp2f(a.part_ml[prow * 2] - M);
      L += a.part_ml[prow * 2 + 1] * w;
      const f32x4 po = *reinterpret_cast<const f32x4 *>(a.part_o + prow * D + d4 * 4);
      acc += po * w;
    }
    const float inv = 1.f / L;
    const int hq = h * a.G + g;
    T *op = reinterpret_cast<T *>(a.out) + (int64_t)b * a.os[0] + (int64_t)qi * a.os[1] +
            (int64_t)hq * a.os[2] + d4 * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) op[e] = (T)(acc[e] * inv);
    if (a.lse && d4 == 0) a.lse[((int64_t)b * a.Hq + hq) * a.q + qi] = (M + __log2f(L)) * kLn2;
  }
}

// -------------------------------------------------------------- general path
// One block per (row, query head, 32-query tile); 8 lanes per query, each
// lane owning D/8 dimensions.  fp32 arithmetic throughout; used for fp32
// inputs and for shapes the MFMA path is not built for.
constexpr int kGenKeys = 32;

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnArgs a) {
  constexpr int DL = D / 8;  // dims per lane
  __shared__ float Kt[kGenKeys][D + 1];
  __shared__ float Vt_[kGenKeys][D + 1];
  const int tid = threadIdx.x;
  const int ql = tid >> 3;   // query inside tile
  const int sub = tid & 7;   // dimension slice
  const int nqt = a.nqt;
  int unit = blockIdx.x;
  const int u = unit % nqt;
  unit /= nqt;
  const int hq = unit % a.Hq;
  const int rl = unit / a.Hq;
  const int b = a.row_ids ? a.row_ids[rl] : rl;
  if (b < 0 || b >= a.B) return;
  const int h = hq / a.G;
  const int P = clampi(a.p_len[b], 0, min(a.p_max, a.p_cap));
  const int qi = u * kQT + ql;
  const bool q_ok = qi < a.q;
  const int ilast = min(u * kQT + kQT, a.q) - 1;
  const int win_len = window_limit(ilast, a.bl, a.q);
  const int lim_i = window_limit(q_ok ? qi : ilast, a.bl, a.q);

  float qv[DL], o[DL];
  const T *qp = reinterpret_cast<const T *>(a.Q) + (int64_t)b * a.qs[0] + (int64_t)qi * a.qs[1] +
                (int64_t)hq * a.qs[2] + sub * DL;
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    qv[e] = q_ok ? (float)qp[e] : 0.f;
    o[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const T *pkb = reinterpret_cast<const T *>(a.pk) + (int64_t)b * a.ps[0] + (int64_t)h * a.ps[2];
  const T *pvb = reinterpret_cast<const T *>(a.pv) + (int64_t)b * a.ps[0] + (int64_t)h * a.ps[2];
  const T *wkb = reinterpret_cast<const T *>(a.wk) + (int64_t)b * a.ws[0] + (int64_t)h * a.ws[2];
  const T *wvb = reinterpret_cast<const T *>(a.wv) + (int64_t)b * a.ws[0] + (int64_t)h * a.ws[2];
  const int npt = (int)cdiv(P, kGenKeys);
  const int nwt = (int)cdiv(win_len, kGenKeys);
  for (int tile = 0; tile < npt + nwt; ++tile) {
    const bool win = tile >= npt;
    const int base = win ? (tile - npt) * kGenKeys : tile * kGenKeys;
    const int limit = win ? win_len : P;
    const T *kb = win ? wkb : pkb;
    const T *vb = win ? wvb : pvb;
    const int64_t sp = win ? a.ws[1] : a.ps[1];
    __syncthreads();
    for (int e = tid; e < kGenKeys * D; e += 256) {
      const int key = e / D, dd = e - key * D;
      const int gk = base + key;
      const bool ok = gk < limit;
      Kt[key][dd] = ok ? (float)kb[(int64_t)gk * sp + dd] : 0.f;
      Vt_[key][dd] = ok ? (float)vb[(int64_t)gk * sp + dd] : 0.f;
    }
    __syncthreads();
    const int vlim = win ? lim_i : limit;
    const int nk = min(kGenKeys, limit - base);
    for (int key = 0; key < nk; ++key) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DL; ++e) dot += qv[e] * Kt[key][sub * DL + e];
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      dot += __shfl_xor(dot, 4);
      if (base + key >= vlim) continue;  // uniform over the 8 lanes of a query
      const float sc = dot * a.scale2;
      const float m_new = fmaxf(m_run, sc);
      const float alpha = exp2f(m_run - m_new);
      const float p = exp2f(sc - m_new);
      l_run = l_run * alpha + p;
#pragma unroll
      for (int e = 0; e < DL; ++e) o[e] = o[e] * alpha + p * Vt_[key][sub * DL + e];
      m_run = m_new;
    }
  }
  if (!q_ok) return;
  T *op = reinterpret_cast<T *>(a.out) + (int64_t)b * a.os[0] + (int64_t)qi * a.os[1] +
          (int64_t)hq * a.os[2] + sub * DL;
  const float inv = 1.f / l_run;
#pragma unroll
  for (int e = 0; e < DL; ++e) op[e] = (T)(o[e] * inv);
  if (a.lse && sub == 0) a.lse[((int64_t)b * a.Hq + hq) * a.q + qi] = (m_run + log2f(l_run)) * kLn2;
}

}  // namespace

bool attn_mfma_supported(int dtype, int d, int G) {
  return dtype == BD_BF16 && d == kD && (G == 1 || G == 2 || G == 4 || G == 8);
}

bool attn_generic_supported(int dtype, int d) {
  return (dtype == BD_BF16 || dtype == BD_F32) && (d == 64 || d == 128);
}

void attn_plan(int dtype, int B, int Hq, int Hkv, int d, int q, int n_rows, int p_max,
               int *chunk, int *n_split, int *nqt, size_t *ws_bytes) {
  (void)B;
  const int G = Hkv > 0 ? Hq / Hkv : 1;
  *nqt = (int)cdiv(q, kQT);
  *chunk = 1 << 30;
  *n_split = 1;
  *ws_bytes = 0;
  if (!attn_mfma_supported(dtype, d, G) || p_max <= 0) return;
  const int64_t units = (int64_t)n_rows * Hkv * (*nqt);
  const int64_t target = 1024;  // blocks wanted to fill 256 CUs a few times
  if (units >= target / 2) return;
  int64_t want = cdiv(target, units);
  const int64_t max_split = cdiv(p_max, kTileK);
  if (want > max_split) want = max_split;
  if (want <= 1) return;
  int64_t ch = cdiv(cdiv(p_max, want), kTileK) * kTileK;
  *chunk = (int)ch;
  *n_split = (int)cdiv(p_max, ch);
  if (*n_split <= 1) {
    *chunk = 1 << 30;
    *n_split = 1;
    return;
  }
  const int64_t prows = units * (*n_split) * G * kQT;
  *ws_bytes = align256((size_t)prows * d * sizeof(float)) + align256((size_t)prows * 2 * sizeof(float));
}

hipError_t launch_attn(const AttnArgs &a_in, hipStream_t s) {
  AttnArgs a = a_in;
  if (attn_mfma_supported(a.dtype, a.d, a.G)) {
    const int64_t n_groups = (int64_t)a.n_rows * a.Hkv;
    const int64_t per_group = (int64_t)a.nqt * a.n_split;
    const int64_t grid = 8 * cdiv(n_groups, 8) * per_group;
    switch (a.G) {
      case 1: hipLaunchKernelGGL(attn_mfma_kernel<1>, dim3((unsigned)grid), dim3(64), 0, s, a); break;
      case 2: hipLaunchKernelGGL(attn_mfma_kernel<2>, dim3((unsigned)grid), dim3(128), 0, s, a); break;
      case 4: hipLaunchKernelGGL(attn_mfma_kernel<4>, dim3((unsigned)grid), dim3(256), 0, s, a); break;
      case 8: hipLaunchKernelGGL(attn_mfma_kernel<8>, dim3((unsigned)grid), dim3(512), 0, s, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split <= 1) return e;
    const int64_t units = n_groups * a.nqt;
    hipLaunchKernelGGL(attn_combine_kernel<bf16>, dim3((unsigned)units), dim3(256), 0, s, a, a.d);
    return hipGetLastError();
  }
  const int64_t grid = (int64_t)a.n_rows * a.Hq * a.nqt;
  if (a.dtype == BD_F32) {
    if (a.d == 64) hipLaunchKernelGGL((attn_generic_kernel<float, 64>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_generic_kernel<float, 128>), dim3((unsigned)grid), dim3(256), 0, s, a);
  } else {
    if (a.d == 64) hipLaunchKernelGGL((attn_generic_kernel<bf16, 64>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_generic_kernel<bf16, 128>), dim3((unsigned)grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bd
