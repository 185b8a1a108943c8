// Fused cache producer (Flash-dLLM, Flash-Cache): the projection of the
// window's hidden states onto the query, key and value heads, the rotary
// embedding of queries and keys at their absolute positions (HERALD Eq. (1);
// FlowBlock's packed windows use absolute positions), and the write of keys
// and values into the cache, with no intermediate tensor in HBM.
//
// One block computes two heads (2 x 128 output features) for 256 window
// tokens: Y^T = W_head X^T with v_mfma_f32_32x32x16_bf16, features on M and
// tokens on N, so a lane ends with 16 features of one token; dimension j and
// its rotary partner j + 64 sit in the same lane and register (M blocks mb
// and mb + 2).  Eight waves: four per head, each owning 64 tokens and the
// head's 128 features (8 MFMAs per 6 fragment reads); every staged X tile
// feeds both heads.  Tiles of 32 hidden elements of W and X are
// double-buffered in LDS and staged through two register sets, so a tile's
// global loads have two tiles of MFMAs to land; one barrier per tile.  The
// rotation angle is formed and reduced to [-pi, pi] in double precision
// (positions reach 1e5 and more; the inverse frequencies come from the host
// in double), its sine and cosine taken in fp32 and applied to the fp32
// accumulators; results are rounded to bf16 once.
#include "bd_common.h"

namespace bd {

namespace {

constexpr int kPD = 128;               // head dim
constexpr int kPTok = 256;             // tokens per block
constexpr int kPBK = 32;               // hidden elements per staged tile
constexpr int kPStr = kPBK;            // LDS row stride (elements): 64 bytes

// LDS element offset of 16-byte chunk c (0..3) of staged row `row`: the chunk
// index is XORed with bits 2-3 of the row, so 16 lanes writing 4 rows x 4
// chunks, and 16 lanes reading one chunk of 16 consecutive rows, each touch
// 16 distinct 4-bank groups of the 64 LDS banks.
__device__ inline int lds_off(int row, int c) { return row * kPStr + ((c ^ ((row >> 2) & 3)) << 3); }

__global__ __launch_bounds__(512, 1) void produce_kernel(ProduceArgs a) {
  const int nheads = a.Hq + 2 * a.Hkv;
  const int t0 = blockIdx.y * kPTok;
  const int tid = threadIdx.x, lane = tid & 63, wave_all = tid >> 6;
  const int hsel = wave_all >> 2, wave = wave_all & 3;   // head of the pair, token quarter
  const int head = min(2 * (int)blockIdx.x + hsel, nheads - 1);
  const bool head_ok = 2 * (int)blockIdx.x + hsel < nheads;
  const int hh = lane >> 5, ln = lane & 31;
  const int n_tok = a.B * a.q;
  __shared__ __attribute__((aligned(16))) bf16 Ws[2][2 * kPD * kPStr];
  __shared__ __attribute__((aligned(16))) bf16 Xs[2][kPTok * kPStr];

  // staging: piece p of a tile is row p / 4, 16-byte chunk p % 4; a thread
  // stages W rows tid/4 and tid/4 + 128 (the pair's two heads) and X rows
  // tid/4 and tid/4 + 128; tokens past the end re-read the last token (their
  // results are not stored)
  const int srow = tid >> 2, kc = tid & 3, kq = kc * 8;   // srow < 128
  // W rows srow and srow + 128 of the pair's 256 (a missing second head
  // re-reads the last head; its results are not stored)
  const bf16 *wrow0 = a.w + ((int64_t)(2 * blockIdx.x) * kPD + srow) * a.Dm + kq;
  const bf16 *wrow1 = a.w + ((int64_t)min(2 * (int)blockIdx.x + 1, nheads - 1) * kPD + srow) * a.Dm + kq;
  const bf16 *xr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int T = min(t0 + srow + 128 * u, n_tok - 1);
    const int b = T / a.q, i = T - b * a.q;
    xr[u] = a.x + (int64_t)b * a.xs[0] + (int64_t)i * a.xs[1] + kq;
  }
  // two register sets: tile it+2 is loaded while tile it is computed and
  // tile it+1 goes from registers to LDS (loads are unconditional, clamped
  // to the last tile, so every wait count is static)
  bf16x8 rw[2][2], rx[2][2];
  const int nit = a.Dm / kPBK;   // even: the loop body handles two tiles
  auto load = [&](int tile, int set) {
    const int k0 = min(tile, nit - 1) * kPBK;
    rw[set][0] = *reinterpret_cast<const bf16x8 *>(wrow0 + k0);
    rw[set][1] = *reinterpret_cast<const bf16x8 *>(wrow1 + k0);
#pragma unroll
    for (int u = 0; u < 2; ++u) rx[set][u] = *reinterpret_cast<const bf16x8 *>(xr[u] + k0);
  };
  auto store = [&](int buf, int set) {
#pragma unroll
    for (int u = 0; u < 2; ++u) *reinterpret_cast<bf16x8 *>(&Ws[buf][lds_off(srow + 128 * u, kc)]) = rw[set][u];
#pragma unroll
    for (int u = 0; u < 2; ++u) *reinterpret_cast<bf16x8 *>(&Xs[buf][lds_off(srow + 128 * u, kc)]) = rx[set][u];
  };

  // acc[nb][mb]: token block nb (32 tokens) x feature block mb (32 features)
  f32x16 acc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x16{};
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kPBK / 16; ++ks) {
      bf16x8 xf[2], wf[4];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        xf[nb] = *reinterpret_cast<const bf16x8 *>(&Xs[buf][lds_off(wave * 64 + nb * 32 + ln, ks * 2 + hh)]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        wf[mb] = *reinterpret_cast<const bf16x8 *>(&Ws[buf][lds_off(hsel * kPD + mb * 32 + ln, ks * 2 + hh)]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[mb], xf[nb], acc[nb][mb], 0, 0, 0);
    }
  };
  load(0, 0);
  store(0, 0);
  load(1, 1);
  load(2, 0);
  __syncthreads();
  for (int it = 0; it < nit; it += 2) {
    compute(0);          // tile it
    store(1, 1);         // tile it + 1
    load(it + 3, 1);
    __syncthreads();
    compute(1);          // tile it + 1
    store(0, 0);         // tile it + 2
    load(it + 4, 0);
    __syncthreads();
  }

  // ---- epilogue: lane holds features mb*32 + (r/4)*8 + hh*4 + r%4 of token T
  if (!head_ok) return;
  const int kind = head < a.Hq ? 0 : (head < a.Hq + a.Hkv ? 1 : 2);   // q, k, v
  constexpr double kTwoPi = 6.283185307179586476925;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int T = t0 + wave * 64 + nb * 32 + ln;
    if (T >= n_tok) continue;
    const int b = T / a.q, i = T - b * a.q;
    if (kind < 2) {
      const double pos = (double)a.rope_pos[b] + (double)i;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int f = mb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
          // angle in double, reduced to [-pi, pi] in double, then sin / cos in fp32
          const double ang = pos * a.inv_freq[f];
          const double red = __builtin_fma(-__builtin_rint(ang * (1.0 / kTwoPi)), kTwoPi, ang);
          float s, c;
          __sincosf((float)red, &s, &c);
          const float lo = acc[nb][mb][r], hi = acc[nb][mb + 2][r];
          acc[nb][mb][r] = lo * c - hi * s;
          acc[nb][mb + 2][r] = hi * c + lo * s;
        }
    }
    bf16 *dst;
    if (kind == 0) {
      dst = a.qo + (int64_t)b * a.qos[0] + (int64_t)i * a.qos[1] + (int64_t)head * a.qos[2];
    } else {
      const int p = a.dst_pos[b] + i;
      if (p < 0 || p >= a.c_cap) continue;   // outside the cache: not written
      const int h = kind == 1 ? head - a.Hq : head - a.Hq - a.Hkv;
      dst = (kind == 1 ? a.kc : a.vc) + (int64_t)b * a.cs[0] + (int64_t)p * a.cs[1] + (int64_t)h * a.cs[2];
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)acc[nb][mb][r4 * 4 + e];
        *reinterpret_cast<bf16x4 *>(dst + mb * 32 + r4 * 8 + hh * 4) = v;
      }
  }
}

}  // namespace

hipError_t launch_produce(const ProduceArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(a.Hq + 2 * a.Hkv, 2), (unsigned)cdiv((int64_t)a.B * a.q, kPTok));
  hipLaunchKernelGGL(produce_kernel, grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace bd
