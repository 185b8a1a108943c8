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
// and mb + 2).  Eight waves, two per SIMD (one wave alone cannot issue MFMAs
// back to back): wave (head h, token quarter t) owns the head's 128 features
// x 64 tokens, 8 accumulators, so each MFMA costs three quarters of an LDS
// fragment read.  Tiles of 64 hidden elements of W and X are double-buffered
// in LDS (128 KB) and reach it by buffer-to-LDS transfers (no staging
// registers, no LDS store instructions): while a tile's 32 MFMAs per wave
// run, the next tile's transfers are in flight.  One block barrier per tile,
// placed before the tile's last 8 MFMAs: after it the next tile's first
// fragments are read and the transfers of the tile after it are issued into
// the buffer just released, under those 8 MFMAs.  Blocks are
// ordered so that the 32 running on one XCD (dispatch is round-robin over
// the 8 XCDs) share 4 head pairs and 8 token tiles, which their L2 serves.
//
// Epilogue: the rotation angle is formed in double as revolutions
// (position x inverse frequency / 2 pi; positions reach 1e5 and more, the
// inverse frequencies come from the host in double), reduced to [-1/2, 1/2]
// in double, and its sine and cosine taken by the hardware's
// revolution-scaled sin / cos in fp32.  A lane's two tokens are 32 apart;
// when all of a wave's lanes hold two consecutive positions of one row
// (always when the window length is a multiple of 64), only the first angle
// is formed that way and the second advances it by the fixed rotation of 32
// positions (cos, sin of 32 x inverse frequency, computed on the host in
// double): one complex product in fp32 in place of a double-precision
// reduction and two sin / cos.  The rotation is applied to the fp32
// accumulators, results are rounded to bf16 once and written, per 32 x 32
// block pair, into the wave's own 16 KB of the (now idle) LDS; read back
// token-major, every store instruction writes whole 256-byte head rows of 4
// tokens (streaming stores: nothing in this launch reads them).  Each of the
// three variants (no rotation, per-angle, stepped) is one straight-line pass
// over the accumulators, so none of them keeps more than one block pair
// outside the accumulator registers.
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

// Rotation (ROT) of the lane's accumulators and their bf16 rows into the
// wave's transpose buffer tw: [32 NB tokens][128 features], 16-byte chunk c of
// token row t at chunk c ^ (t & 15), the 8-byte halves swapped for rows with
// bit 4 set, so the 32 lanes of one write (rows 0..31) spread over all 64
// banks.  Lane (hh, ln) holds features mb*32 + g*8 + hh*4 + e (r = 4g + e)
// of token nb*32 + ln; dimension j and its partner j + 64 are blocks mb and
// mb + 2 of the same register.  STEP: the angle of each token nb > 0
// advances that of token nb - 1 by the rotation of 32 positions.
template <bool ROT, bool STEP, int NB>
__device__ __forceinline__ void rope_to_lds(f32x16 (&acc)[NB][4], bf16 *tw, const double (&pos)[NB],
                                            const ProduceArgs &a, int hh, int ln) {
  constexpr double kRev = 0.15915494309189533577;   // 1 / (2 pi)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    double fr[16];   // revolutions per position of the lane's dimensions
    float stc[16], sts[16];
    float cs[16], sn[16];
    if (ROT) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = mb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
        fr[r] = a.inv_freq[j] * kRev;
        if (STEP) { stc[r] = a.step_rot[j][0]; sts[r] = a.step_rot[j][1]; }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float lo[16], hi[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) { lo[r] = acc[nb][mb][r]; hi[r] = acc[nb][mb + 2][r]; }
      if (ROT) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (STEP && nb > 0) {
            const float c0 = cs[r], s0 = sn[r];
            cs[r] = c0 * stc[r] - s0 * sts[r];
            sn[r] = s0 * stc[r] + c0 * sts[r];
          } else {
            const double x = pos[nb] * fr[r];
            const float t = (float)(x - __builtin_rint(x));   // [-1/2, 1/2] revolutions
            sn[r] = __builtin_amdgcn_sinf(t);
            cs[r] = __builtin_amdgcn_cosf(t);
          }
          const float l = lo[r], h = hi[r];
          lo[r] = l * cs[r] - h * sn[r];
          hi[r] = h * cs[r] + l * sn[r];
        }
      }
      const int row = nb * 32 + ln;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v, u;
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = (bf16)lo[g * 4 + e]; u[e] = (bf16)hi[g * 4 + e]; }
        const int sw = (hh ^ (ln >> 4)) << 2;
        *reinterpret_cast<bf16x4 *>(&tw[row * kPD + (((mb * 4 + g) ^ (row & 15)) << 3) + sw]) = v;
        *reinterpret_cast<bf16x4 *>(&tw[row * kPD + ((((mb + 2) * 4 + g) ^ (row & 15)) << 3) + sw]) = u;
      }
    }
  }
}

__global__ __launch_bounds__(512, 1) void produce_kernel(ProduceArgs a, int n_pairs, int n_tb, int xcd_order) {
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
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hsel = wave >> 2, tq = wave & 3;   // head of the pair, token quarter
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

  // staging by buffer-to-LDS transfers: wave w fills the 1 KB blocks
  // gb = 8 (w % 4) + p (p < 8) of W (waves 0-3: the pair's 256 feature rows;
  // a missing second head re-reads the last head) or of X (waves 4-7: tokens
  // past the end re-read the last token), rows 8 gb .. 8 gb + 7; lane l
  // writes chunk position l % 8 of row 8 gb + l / 8 and loads into it the
  // global chunk (l % 8) ^ ((row / 2) % 8), the swizzle of lds_off
  const bool isx = wave >= 4;
  int voff[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int gb = 8 * (wave & 3) + p, row = 8 * gb + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    if (!isx) {
      const int hd = min(2 * pair + (row >> 7), nheads - 1);
      voff[p] = (int)((((int64_t)hd * kPD + (row & 127)) * a.Dm + c * 8) * 2);
    } else {
      const int T = min(t0 + row, n_tok - 1);
      const int b = T / a.q, i = T - b * a.q;
      voff[p] = (int)(((int64_t)b * a.xs[0] + (int64_t)i * a.xs[1] + c * 8) * 2);
    }
  }
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)(isx ? a.x : a.w), (short)0, 0x7fffffff, 0x00020000);
  const int nit = a.Dm / kPBK;
  auto dma = [&](bf16 *Wn, bf16 *Xn, int k0) __attribute__((always_inline)) {
    bf16 *dst = isx ? Xn : Wn;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int gb = 8 * (wave & 3) + p;
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)&dst[gb * 512], 16,
                                               voff[p], k0 * 2, 0, 0);
#else
      (void)dst, (void)gb, (void)k0;   // the builtin exists in the device pass only
#endif
    }
  };

  // acc[nb][mb]: token block nb (32 tokens) x feature block mb (32 features)
  f32x16 acc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x16{};
  auto frag = [&](const bf16 *Wb, const bf16 *Xb, int ks, bf16x8 *xf, bf16x8 *wf) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      xf[nb] = *reinterpret_cast<const bf16x8 *>(&Xb[lds_off(tq * 64 + nb * 32 + ln, ks * 2 + hh)]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      wf[mb] = *reinterpret_cast<const bf16x8 *>(&Wb[lds_off(hsel * kPD + mb * 32 + ln, ks * 2 + hh)]);
  };
  // One tile from (Wb, Xb), whose successor is already in flight into
  // (Wn, Xn).  Steps 0-2 (16 elements each): 8 MFMAs and the next step's 6
  // fragment reads.  The block barrier (which waits for every wave's
  // transfers into (Wn, Xn)) then comes before step 3: the tile's last
  // fragments are in registers, so (Wb, Xb) is free; the next tile's first
  // fragments are read and the transfers of the tile after it into (Wb, Xb)
  // are issued while step 3's MFMAs run.
  bf16x8 xf[2][2], wf[2][4];
  auto mfma8 = [&](int b) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[b][mb], xf[b][nb], acc[nb][mb], 0, 0, 0);
  };
  auto step = [&](bf16 *Wb, bf16 *Xb, const bf16 *Wn, const bf16 *Xn, int t_refill) {
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      frag(Wb, Xb, ks + 1, xf[(ks + 1) & 1], wf[(ks + 1) & 1]);
      mfma8(ks & 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // this wave's transfers into (Wn, Xn) have landed (the transfers count
    // on the vector memory counter), then every wave's
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    frag(Wn, Xn, 0, xf[0], wf[0]);
    if (t_refill < nit) dma(Wb, Xb, t_refill * kPBK);
    mfma8(1);
  };
  dma(W0, X0, 0);
  if (nit > 1) dma(W1, X1, kPBK);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  frag(W0, X0, 0, xf[0], wf[0]);
  for (int it = 0; it < nit; it += 2) {
    step(W0, X0, W1, X1, it + 2);
    if (it + 1 < nit) step(W1, X1, W0, X0, it + 3);   // odd tile count
  }

  // ---- epilogue: lane holds features mb*32 + g*8 + hh*4 + e (r = 4g + e) of
  // token nb*32 + ln of its quarter
  if (!head_ok) return;
  // the lane's indices formed again from the execution mask (nothing
  // derived from the thread index is kept across the loop)
  const int el = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int ehh = el >> 5, eln = el & 31;
  const int kind = head < a.Hq ? 0 : (head < a.Hq + a.Hkv ? 1 : 2);   // q, k, v
  bf16 *const tb2 = (wave >> 1) == 0 ? W0 : ((wave >> 1) == 1 ? W1 : ((wave >> 1) == 2 ? X0 : X1));
  bf16 *const tw = tb2 + (wave & 1) * (64 * kPD);
  double pos[2];
  bool step_ok = true;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int T = min(t0 + tq * 64 + nb * 32 + eln, n_tok - 1);
    const int b = T / a.q, i = T - b * a.q;
    pos[nb] = (double)a.rope_pos[b] + (double)i;
    step_ok = step_ok && pos[nb] == pos[0] + 32.0 * nb;
  }
  // the three variants are chosen per wave (uniform branches)
  if (kind == 2) rope_to_lds<false, false, 2>(acc, tw, pos, a, ehh, eln);
  else if (__all(step_ok)) rope_to_lds<true, true, 2>(acc, tw, pos, a, ehh, eln);
  else rope_to_lds<true, false, 2>(acc, tw, pos, a, ehh, eln);
  // the wave reads what its other lanes wrote: LDS completes a wave's
  // accesses in order; the fences keep the compiler from reordering them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int c16 = el & 15;
  const float inv_q = 1.f / (float)a.q;
  const int hk = kind == 1 ? head - a.Hq : head - a.Hq - a.Hkv;
  bf16 *const cache = kind == 1 ? a.kc : a.vc;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = j * 4 + (el >> 4);   // bit 4 of row is bit 2 of j
    bf16x8 v = *reinterpret_cast<const bf16x8 *>(&tw[row * kPD + ((c16 ^ (row & 15)) << 3)]);
    if (j & 4) v = __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3);
    const int T = t0 + tq * 64 + row;
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
    typedef int i32x4v __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(i32x4v, v), reinterpret_cast<i32x4v *>(dst + c16 * 8));
  }
}

}  // namespace

hipError_t launch_produce(const ProduceArgs &args, hipStream_t s) {
  ProduceArgs a = args;
  for (int j = 0; j < 64; ++j) {
    a.step_rot[j][0] = (float)cos(32.0 * a.inv_freq[j]);
    a.step_rot[j][1] = (float)sin(32.0 * a.inv_freq[j]);
  }
  const int n_pairs = (int)cdiv(a.Hq + 2 * a.Hkv, 2), n_tb = (int)cdiv((int64_t)a.B * a.q, kPTok);
  const int total = n_pairs * n_tb;
  hipLaunchKernelGGL(produce_kernel, dim3((unsigned)total), dim3(512), 0, s, a, n_pairs, n_tb,
                     total % 8 == 0 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace bd
