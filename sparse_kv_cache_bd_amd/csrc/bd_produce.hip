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
// and mb + 2).  Four waves, one per SIMD: wave (head h, token half t) owns
// the head's 128 features x 128 tokens, 16 accumulators in AGPRs, so each
// MFMA costs half an LDS fragment read.  Tiles of 64 hidden elements of W and
// X are double-buffered in LDS (128 KB); while a tile's 64 MFMAs run, the
// next tile goes from registers to the other buffer and the tile after it is
// loaded into the registers, the three interleaved one-for-one with the
// MFMAs by scheduling barriers.  One block barrier per tile.  Blocks are
// ordered so that the 32 running on one XCD (dispatch is round-robin over
// the 8 XCDs) share 4 head pairs and 8 token tiles, which their L2 serves.
//
// Epilogue: the rotation angle is formed in double as revolutions
// (position x inverse frequency / 2 pi; positions reach 1e5 and more, the
// inverse frequencies come from the host in double), reduced to [-1/2, 1/2]
// in double, and its sine and cosine taken by the hardware's
// revolution-scaled sin / cos in fp32; the rotation is applied to the fp32
// accumulators and results are rounded to bf16 once.  Each wave then writes
// its 128 x 128 tile into its own 32 KB of the (now idle) LDS and reads it
// back token-major, so every store instruction writes whole 256-byte head
// rows of 4 tokens.
#include "bd_common.h"

namespace bd {

namespace {

constexpr int kPD = 128;     // head dim
constexpr int kPTok = 256;   // tokens per block
constexpr int kPBK = 64;     // hidden elements per staged tile
constexpr int kPStr = kPBK;  // LDS row stride (elements): 128 bytes
constexpr int kPGroup = 4;   // head pairs per group of the block order

// LDS element offset of 16-byte chunk c (0..7) of staged row `row`: the chunk
// index is XORed with bits 1-3 of the row, so 16 lanes writing 2 rows x 8
// chunks, and 16 lanes reading one chunk of 16 consecutive rows, each touch
// 16 distinct 4-bank groups of the 64 LDS banks.
__device__ inline int lds_off(int row, int c) { return row * kPStr + ((c ^ ((row >> 1) & 7)) << 3); }

__global__ __launch_bounds__(256, 1) void produce_kernel(ProduceArgs a, int n_pairs, int n_tb, int xcd_order) {
  // block -> (head pair, token tile): with xcd_order, XCD x (= blockIdx % 8)
  // runs the contiguous eighth x of the tiles; tiles run in groups of
  // kPGroup head pairs, token tiles outer, so concurrent blocks share operands
  int tile = blockIdx.x;
  if (xcd_order) tile = (tile & 7) * ((n_pairs * n_tb) >> 3) + (tile >> 3);
  const int g0 = (tile / (kPGroup * n_tb)) * kPGroup;
  const int gl = min(kPGroup, n_pairs - g0);
  const int gi = tile - g0 * n_tb;
  const int tb = gi / gl, pair = g0 + gi % gl;

  const int nheads = a.Hq + 2 * a.Hkv;
  const int t0 = tb * kPTok;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hsel = wave >> 1, tq = wave & 1;   // head of the pair, token half
  const int head = min(2 * pair + hsel, nheads - 1);
  const bool head_ok = 2 * pair + hsel < nheads;
  const int hh = lane >> 5, ln = lane & 31;
  const int n_tok = a.B * a.q;
  // separate arrays per buffer: the compiler sees that the staging writes
  // into one buffer never alias the fragment reads of the other
  __shared__ __attribute__((aligned(16))) bf16 W0[2 * kPD * kPStr];
  __shared__ __attribute__((aligned(16))) bf16 W1[2 * kPD * kPStr];
  __shared__ __attribute__((aligned(16))) bf16 X0[kPTok * kPStr];
  __shared__ __attribute__((aligned(16))) bf16 X1[kPTok * kPStr];

  // staging: thread tid holds chunk kc of rows srow + 32u (u < 8) of both the
  // W tile (the pair's 256 feature rows; a missing second head re-reads the
  // last head, its results are not stored) and the X tile (tokens past the
  // end re-read the last token, their results are not stored)
  const int srow = tid >> 3, kc = tid & 7, kq = kc * 8;
  const bf16 *wrow[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    wrow[h] = a.w + ((int64_t)min(2 * pair + h, nheads - 1) * kPD + srow) * a.Dm + kq;
  const bf16 *xr[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int T = min(t0 + srow + 32 * u, n_tok - 1);
    const int b = T / a.q, i = T - b * a.q;
    xr[u] = a.x + (int64_t)b * a.xs[0] + (int64_t)i * a.xs[1] + kq;
  }
  bf16x8 rg[16];   // units 0..7: W rows srow + 32u; 8..15: X rows srow + 32(u - 8)
  const int nit = a.Dm / kPBK;
  auto gload = [&](int u, int k0) {
    if (u < 8) rg[u] = *reinterpret_cast<const bf16x8 *>(wrow[u >> 2] + (int64_t)(32 * (u & 3)) * a.Dm + k0);
    else rg[u] = *reinterpret_cast<const bf16x8 *>(xr[u - 8] + k0);
  };
  auto lstore = [&](bf16 *Wn, bf16 *Xn, int u) {
    if (u < 8) *reinterpret_cast<bf16x8 *>(&Wn[lds_off(srow + 32 * u, kc)]) = rg[u];
    else *reinterpret_cast<bf16x8 *>(&Xn[lds_off(srow + 32 * (u - 8), kc)]) = rg[u];
  };

  // acc[nb][mb]: token block nb (32 tokens) x feature block mb (32 features)
  f32x16 acc[4][4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x16{};
  auto frag = [&](const bf16 *Wb, const bf16 *Xb, int ks, bf16x8 *xf, bf16x8 *wf) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      xf[nb] = *reinterpret_cast<const bf16x8 *>(&Xb[lds_off(tq * 128 + nb * 32 + ln, ks * 2 + hh)]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      wf[mb] = *reinterpret_cast<const bf16x8 *>(&Wb[lds_off(hsel * kPD + mb * 32 + ln, ks * 2 + hh)]);
  };
  // One tile from (Wb, Xb); the registers' tile goes to (Wn, Xn) and the tile
  // at hidden offset k0 is loaded.  Per 16-element step: 16 MFMAs, the next
  // step's 8 fragment reads, 4 staging writes and 4 global loads.
  auto step = [&](const bf16 *Wb, const bf16 *Xb, bf16 *Wn, bf16 *Xn, int k0) {
    bf16x8 xf[2][4], wf[2][4];
    frag(Wb, Xb, 0, xf[0], wf[0]);
#pragma unroll
    for (int ks = 0; ks < kPBK / 16; ++ks) {
      if (ks < kPBK / 16 - 1) frag(Wb, Xb, ks + 1, xf[(ks + 1) & 1], wf[(ks + 1) & 1]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lstore(Wn, Xn, 4 * ks + j);
        gload(4 * ks + j, k0);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][mb], xf[ks & 1][nb], acc[nb][mb], 0, 0, 0);
      // masks: 0x008 MFMA, 0x020 global load, 0x100 LDS read, 0x200 LDS write
      if (ks < kPBK / 16 - 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
      }
    }
    __syncthreads();
  };
  // loads past the last tile are clamped to it (their data is never used),
  // so every wait count is static
#pragma unroll
  for (int u = 0; u < 16; ++u) gload(u, 0);
#pragma unroll
  for (int u = 0; u < 16; ++u) lstore(W0, X0, u);
#pragma unroll
  for (int u = 0; u < 16; ++u) gload(u, min(1, nit - 1) * kPBK);
  __syncthreads();
  int it = 0;
  for (; it + 1 < nit; it += 2) {
    step(W0, X0, W1, X1, min(it + 2, nit - 1) * kPBK);
    step(W1, X1, W0, X0, min(it + 3, nit - 1) * kPBK);
  }
  if (it < nit) step(W0, X0, W1, X1, (nit - 1) * kPBK);   // odd tile count

  // ---- epilogue: lane holds features mb*32 + g*8 + hh*4 + e (r = 4g + e) of
  // token nb*32 + ln of its half
  if (!head_ok) return;
  const int kind = head < a.Hq ? 0 : (head < a.Hq + a.Hkv ? 1 : 2);   // q, k, v
  if (kind < 2) {
    constexpr double kRev = 0.15915494309189533577;   // 1 / (2 pi)
    double pos[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int T = min(t0 + tq * 128 + nb * 32 + ln, n_tok - 1);
      const int b = T / a.q, i = T - b * a.q;
      pos[nb] = (double)a.rope_pos[b] + (double)i;
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      double fr[4][4];   // revolutions per position of the lane's dimensions mb*32 + g*8 + hh*4 + e
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) fr[g][e] = a.inv_freq[mb * 32 + g * 8 + hh * 4 + e] * kRev;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const double x = pos[nb] * fr[r >> 2][r & 3];
          const float t = (float)(x - __builtin_rint(x));   // [-1/2, 1/2] revolutions
          const float s = __builtin_amdgcn_sinf(t), c = __builtin_amdgcn_cosf(t);
          const float lo = acc[nb][mb][r], hi = acc[nb][mb + 2][r];
          acc[nb][mb][r] = lo * c - hi * s;
          acc[nb][mb + 2][r] = hi * c + lo * s;
        }
    }
  }
  // transpose through this wave's 32 KB: [128 tokens][128 features] bf16,
  // 16-byte chunk c of token row t stored at chunk c ^ (t & 15); the 8-byte
  // halves are swapped for rows with bit 4 set, so the 32 lanes of one write
  // (rows 0..31) spread over all 64 banks
  bf16 *const tw = wave == 0 ? W0 : (wave == 1 ? W1 : (wave == 2 ? X0 : X1));
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = nb * 32 + ln;
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)acc[nb][mb][g * 4 + e];
        *reinterpret_cast<bf16x4 *>(&tw[row * kPD + (((mb * 4 + g) ^ (row & 15)) << 3) + ((hh ^ (ln >> 4)) << 2)]) = v;
      }
  // the wave reads what its other lanes wrote: LDS completes a wave's
  // accesses in order; the fences keep the compiler from reordering them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int c16 = lane & 15;
  const float inv_q = 1.f / (float)a.q;
  const int hk = kind == 1 ? head - a.Hq : head - a.Hq - a.Hkv;
  bf16 *const cache = kind == 1 ? a.kc : a.vc;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int row = j * 4 + (lane >> 4);   // bit 4 of row is bit 2 of j
    bf16x8 v = *reinterpret_cast<const bf16x8 *>(&tw[row * kPD + ((c16 ^ (row & 15)) << 3)]);
    if (j & 4) v = __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3);
    const int T = t0 + tq * 128 + row;
    if (T >= n_tok) continue;
    // b = T / q from a float estimate (T < 2^24, checked on the host) and
    // one correction each way
    int b = (int)((float)T * inv_q);
    int i = T - b * a.q;
    if (i < 0) { --b; i += a.q; }
    if (i >= a.q) { ++b; i -= a.q; }
    bf16 *dst;
    if (kind == 0) {
      dst = a.qo + (int64_t)b * a.qos[0] + (int64_t)i * a.qos[1] + (int64_t)head * a.qos[2];
    } else {
      const int p = a.dst_pos[b] + i;
      if (p < 0 || p >= a.c_cap) continue;   // outside the cache: not written
      dst = cache + (int64_t)b * a.cs[0] + (int64_t)p * a.cs[1] + (int64_t)hk * a.cs[2];
    }
    *reinterpret_cast<bf16x8 *>(dst + c16 * 8) = v;
  }
}

}  // namespace

hipError_t launch_produce(const ProduceArgs &a, hipStream_t s) {
  const int n_pairs = (int)cdiv(a.Hq + 2 * a.Hkv, 2), n_tb = (int)cdiv((int64_t)a.B * a.q, kPTok);
  const int total = n_pairs * n_tb;
  hipLaunchKernelGGL(produce_kernel, dim3((unsigned)total), dim3(256), 0, s, a, n_pairs, n_tb,
                     total % 8 == 0 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace bd
