// Block-diffusion attention: GQA, per-row prefix length, W-shaped window mask
// (FlowBlock review Eq. (6)); HERALD's denoising attention over a pool when
// the prefix is a gathered pool.
//
// MFMA path (bf16, d = 128).  A block of NW = 8 waves (two per SIMD, so
// one wave's softmax overlaps the other's MFMAs) owns one (row, KV head,
// query tile, key chunk) work item; 4-wave blocks serve small GQA windows.
// The tile's columns are (query, query head) pairs of the GQA group, 32 per
// wave.  Every column of a block sees the same prefix keys, so one K/V tile
// staged in LDS serves all of them.
//
// Per 64-key tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (keys on M, columns on N): a lane then holds 16 scores of one column, so
// the online softmax (FlashAttention running max / sum) is lane-local, with
// one exchange with lane l^32 for the column max.  O^T += V^T P^T takes the
// S^T accumulator registers directly as the B operand; V stays key-major in
// LDS and its V^T fragments come from transposing LDS reads
// (ds_read_b64_tr_b16), two per fragment, which hand each lane the keys its
// accumulator registers hold.  The running max is only raised when a tile's
// max exceeds it by more than 2^8 (the result is the same for any reference
// value; p stays <= 256), so the O rescale runs on few tiles.
//
// Pipelining: K and V tiles are double-buffered in LDS with one barrier per
// tile; both go from memory straight into LDS (buffer-to-LDS transfers, no
// registers, no LDS store instructions), the transfers of tile t+1 issued
// before the MFMAs of tile t.  Inside a tile the exponentials of the second
// 32-key half are independent of the P V MFMAs of the first half.
//
// Rows at or past the prefix length are never read (the buffer range check
// returns zeros for them, and their scores are masked), which keeps NaN
// sentinels in unused rows out of the arithmetic.
//
// Scheduling: with more work items than the GPU holds at once, a planner
// kernel ranks the rows by prefix length and blocks take rows longest first
// (LPT order).  The items of one (row, KV head) go to the same XCD, so its
// K/V come from HBM into that XCD's L2 once.  With few items the prefix is
// cut into chunks; each chunk writes its normalised partial O (bf16) with
// its (max, sum), and a combine kernel merges the chunks in a fixed order.
#include "bd_common.h"

namespace bd {

namespace {

// ----------------------------------------------------------------- MFMA path
constexpr int kD = 128;            // head dim of the MFMA path
constexpr int kTK = 64;            // keys per staged tile
constexpr int kKRow = kD;          // LDS row of K (elements): 256 B, 16-byte chunks swizzled
constexpr int kKTile = kTK * kKRow;
constexpr int kVTile = kTK * kD;   // key-major V (elements): 256-byte rows, 16-byte chunks swizzled
constexpr float kRescaleSlack = 8.f;  // log2 units

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
struct bf16x2x4 { bf16x2 v[4]; };

__device__ inline bf16x8 ld_bf16x8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Row list position rl -> row and prefix source (the second source holds
// the positions at or past n_rows1).
struct RowRef {
  int b;
  bool alt;
};
__device__ inline RowRef row_ref(const AttnArgs &a, int rl) {
  if (rl < a.n_rows1) return {a.row_ids ? a.row_ids[rl] : rl, false};
  return {a.row_ids2[rl - a.n_rows1], true};
}
// prefix length of a row whose index b is in [0, B)
__device__ inline int prefix_len(const AttnArgs &a, const RowRef &r) {
  return r.alt ? clampi(a.p_len2[r.b], 0, min(a.p_max2, a.p_cap2))
               : clampi(a.p_len[r.b], 0, min(a.p_max, a.p_cap));
}
// Wave-uniform 64-bit value in scalar registers.  Choosing between two
// fields of the argument block through this keeps the choice a select of
// values (a select of the fields' addresses would keep the block in memory).
__device__ inline uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// Prefix source of a row: K, V base of (row b, KV head h) and key row stride.
struct PrefixSrc {
  const char *k, *v;
  int64_t row;
};
__device__ inline PrefixSrc prefix_src(const AttnArgs &a, const RowRef &r, int h, int es) {
  const uint64_t pk = uniform_u64(r.alt ? reinterpret_cast<uint64_t>(a.pk2) : reinterpret_cast<uint64_t>(a.pk));
  const uint64_t pv = uniform_u64(r.alt ? reinterpret_cast<uint64_t>(a.pv2) : reinterpret_cast<uint64_t>(a.pv));
  const int64_t s0 = (int64_t)uniform_u64((uint64_t)(r.alt ? a.ps2[0] : a.ps[0]));
  const int64_t s1 = (int64_t)uniform_u64((uint64_t)(r.alt ? a.ps2[1] : a.ps[1]));
  const int64_t s2 = (int64_t)uniform_u64((uint64_t)(r.alt ? a.ps2[2] : a.ps[2]));
  const int64_t off = ((int64_t)r.b * s0 + (int64_t)h * s2) * es;
  return {reinterpret_cast<const char *>(pk) + off, reinterpret_cast<const char *>(pv) + off, s1};
}

// Block of NW waves, one 32-column group per wave; two waves share a SIMD.
// Tile staging: 16 K and 16 V transfers of 1 KB (memory to LDS) per 64-key
// tile.  With 8 waves, waves 0-3 move V and waves 4-7 K (4 transfers per
// wave); with 4 waves every wave moves 4 of each.
template <int NW, int G>
struct Shape {
  static constexpr int NT = 64 * NW;           // threads
  static constexpr int NCG = NW;               // 32-column groups per block
  static constexpr int QB = NCG / G;           // 32-query blocks per block
  static constexpr int NQ = 32 * QB;           // queries per block
  static constexpr int NCOL = 32 * NCG;        // columns per block
  static constexpr bool SPLIT_STAGE = NW == 8;
  static constexpr int VI = 1;                 // V items per staging thread
  static_assert(QB >= 1 && NCG % G == 0, "GQA group larger than the block");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
};

// Decoded work item of a block.
struct Item {
  RowRef r;
  int b, h, rl, u, c, nc;
  int kbeg, kend;     // prefix keys of this chunk
  bool with_window;   // last chunk also covers the window
  int q0, q1;         // window queries of the item (block-table mode)
  int toff;           // first page-table entry of the item (block-table mode)
};

// Work item of one block-table list position: row, query range, page-table
// offset and key count, validated (an invalid item is skipped).
__device__ inline bool bt_item(const AttnArgs &a, int n, int &b, int &q0, int &q1, int &toff, int &P) {
  const bd_attn_item e = a.items[n];
  b = e.row;
  q0 = e.q_begin;
  q1 = min(e.q_end, a.q);
  toff = e.table_off;
  P = clampi(e.kv_len, 0, a.p_max);
  return b >= 0 && b < a.B && q0 >= 0 && q0 < q1 && toff >= 0 &&
         (int64_t)toff + cdiv(P, a.page) <= a.n_table;
}

template <bool BT>
__device__ inline bool decode_item(const AttnArgs &a, int bid, Item &it, int nq_tile) {
  const int per_group = a.nqt * a.n_split;
  const int xcd = bid & 7;
  const int sigma = bid >> 3;
  const int gamma = xcd + 8 * (sigma / per_group);
  if (gamma >= a.n_rows * a.Hkv) return false;
  const int mem = sigma - (sigma / per_group) * per_group;
  it.u = mem / a.n_split;
  it.c = mem - it.u * a.n_split;
  const int rank = gamma / a.Hkv;
  it.h = gamma - rank * a.Hkv;
  int P;
  if constexpr (BT) {
    // list order is the caller's order: no ranking
    it.rl = rank;
    it.r = RowRef{0, false};
    if (!bt_item(a, rank, it.b, it.q0, it.q1, it.toff, P)) return false;
    if (it.q0 + it.u * nq_tile >= it.q1) return false;
  } else {
    it.rl = a.row_order ? a.row_order[rank] : rank;
    it.r = row_ref(a, it.rl);
    it.b = it.r.b;
    if (it.b < 0 || it.b >= a.B) return false;
    P = prefix_len(a, it.r);
    it.q0 = 0;
    it.q1 = a.q;
    it.toff = 0;
  }
  it.nc = P > 0 ? (int)cdiv(P, a.chunk) : 1;
  if (it.c >= it.nc) return false;
  it.kbeg = it.c * a.chunk;
  it.kend = min(P, it.kbeg + a.chunk);
  it.with_window = (it.c == it.nc - 1);
  return true;
}

// WM: a window mask other than block-causal (a.mask_mode); a separate
// instance, so the block-causal kernel carries none of its code.
// BT: block-table mode (work items over a paged store; bd_attn_block_table).
template <int NW, int G, bool WM, bool BT>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_mfma_kernel(AttnArgs a) {
  using S = Shape<NW, G>;
  // one array per buffer: the compiler then sees that the K transfers into
  // one buffer never alias the fragment reads of the other, and waits for
  // them only at the tile barrier
  __shared__ __attribute__((aligned(16))) bf16 Ks0[kKTile];
  __shared__ __attribute__((aligned(16))) bf16 Ks1[kKTile];
  __shared__ __attribute__((aligned(16))) bf16 Vt0[kVTile];
  __shared__ __attribute__((aligned(16))) bf16 Vt1[kVTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;  // lane half
  const int ln = lane & 31;  // column / M row inside a 32x32 tile

  Item it;
  if (!decode_item<BT>(a, blockIdx.x, it, S::NQ)) return;
  const int b = it.b, h = it.h;
  // queries [q0, q1) of the item (all q window queries outside block-table mode)
  const int q0 = BT ? it.q0 : 0;
  const int q1 = BT ? it.q1 : a.q;
  const int i0 = q0 + it.u * S::NQ;
  const int ilast = min(i0 + S::NQ, q1) - 1;
  const int win_len = window_limit(ilast, a.bl, a.q);
  const int n_pref = it.kend > it.kbeg ? (int)cdiv(it.kend - it.kbeg, kTK) : 0;
  const int n_tiles = n_pref + (it.with_window ? (int)cdiv(win_len, kTK) : 0);

  // ---- this wave's column group: one query head, 32 queries
  const int g = wave / S::QB;
  const int qb = wave - g * S::QB;
  const int hq = h * G + g;
  const int qi = i0 + qb * 32 + ln;
  const bool qok = qi < q1;
  const int lim = window_limit(qok ? qi : ilast, a.bl, a.q);
  // other window masks: window keys in [w_shared, w_floor) are not visible
  const int w_floor = WM ? window_floor(qok ? qi : ilast, a.bl, a.mask_mode) : 0;
  const int w_shared = WM ? window_shared(a.bl, a.mask_mode) : 0;

  // ---- Q operands (B of S^T = K Q^T): lane holds Q[qi][ks*16 + hh*8 .. +8]
  bf16x8 qop[kD / 16];
  {
    const bf16 *qp = reinterpret_cast<const bf16 *>(a.Q) + (int64_t)b * a.qs[0] +
                     (int64_t)(qok ? qi : 0) * a.qs[1] + (int64_t)hq * a.qs[2] + hh * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) qop[ks] = qok ? ld_bf16x8(qp + ks * 16) : bf16x8{};
  }

  // prefix base of (row b, KV head h); in block-table mode the page store's
  // head h (pages are added per tile)
  const PrefixSrc src = BT ? PrefixSrc{reinterpret_cast<const char *>(a.pk) + (int64_t)h * a.ps[2] * 2,
                                       reinterpret_cast<const char *>(a.pv) + (int64_t)h * a.ps[2] * 2,
                                       a.ps[1]}
                           : prefix_src(a, it.r, h, (int)sizeof(bf16));
  const bf16 *pkb = reinterpret_cast<const bf16 *>(src.k);
  const bf16 *pvb = reinterpret_cast<const bf16 *>(src.v);
  const int64_t p_row = src.row, w_row = a.ws[1];   // key row strides
  const bf16 *wkb = reinterpret_cast<const bf16 *>(a.wk) + (int64_t)b * a.ws[0] + (int64_t)h * a.ws[2];
  const bf16 *wvb = reinterpret_cast<const bf16 *>(a.wv) + (int64_t)b * a.ws[0] + (int64_t)h * a.ws[2];

  // tile tt: first key, end of the valid keys, source (prefix or window)
  auto tile_base = [&](int tt) { return tt < n_pref ? it.kbeg + tt * kTK : (tt - n_pref) * kTK; };
  auto tile_limit = [&](int tt) { return tt < n_pref ? it.kend : win_len; };

  // ---- staging with buffer loads.  Each tile gets a buffer resource based
  // at its first key whose size ends at the tile's last valid key, so rows at
  // or past the limit read as zeros (the hardware range check) and unused
  // rows are never touched.  Offsets are 32-bit: one tile spans at most kTK
  // rows (the host checks the row strides).
  // K and V go straight from memory into LDS (buffer-to-LDS transfers):
  // each staging wave moves 4 blocks of 4 key rows, one 1 KB transfer per
  // block; lane l writes the 16 bytes at l * 16 of its block, i.e. chunk
  // l % 16 of row l / 16 in the block, and loads into it a chosen global
  // chunk, which swizzles the rows: chunk c of key row r sits at chunk
  // c ^ (r % 16) for K (the fragment reads of 32 rows spread over the
  // banks) and at c ^ 4 (r % 4) for V (the transposing reads of 4 rows x
  // 4 dims per lane group spread over the banks).
  const bool stage_v = !S::SPLIT_STAGE || wave < 4;
  const bool stage_k = !S::SPLIT_STAGE || wave >= 4;
  auto rsrc = [](const bf16 *p, int64_t row_el, int base, int limit) {
    const int64_t rowb = row_el * 2;
    const int rows = min(limit - base, kTK);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(p + (int64_t)base * row_el), (short)0,
                                             (int)(rows * rowb), 0x00020000);
  };
  // block-table mode: page id of the next prefix tile to load, requested
  // one tile ahead with a buffer load (it waits on the vector memory counter
  // with the K/V loads, not on the LDS counter the tile's fragment reads
  // use); valid rows of the tiles in the two LDS buffers
  int pg_next = 0;
  int rows_buf0 = kTK, rows_buf1 = kTK;
  const auto trsrc = __builtin_amdgcn_make_buffer_rsrc((void *)a.table, (short)0,
                                                       BT ? a.n_table * 4 : 0, 0x00020000);
  auto request_page = [&](int tt) {
    if (BT && tt < n_pref) {
      const int k0 = it.kbeg + tt * kTK;
      pg_next = (int)__builtin_amdgcn_raw_buffer_load_b32(trsrc, (it.toff + k0 / a.page) * 4, 0, 0);
    }
  };
  // per-lane parts of the transfer offsets, fixed over the tiles: lane l
  // fills chunk l % 16 of row 4 blk + l / 16; row r's global chunk c lands at
  // chunk c ^ (r % 16) for K and c ^ 4 (r % 4) for V, and r % 16 =
  // 4 p + l / 16 for transfer p, r % 4 = l / 16
  const int lrow_p = (lane >> 4) * (int)(p_row * 2), lrow_w = (lane >> 4) * (int)(w_row * 2);
  int kchunk[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) kchunk[p] = ((lane & 15) ^ (4 * p + (lane >> 4))) << 4;
  const int vchunk = ((lane & 15) ^ ((lane >> 4) << 2)) << 4;
  auto load = [&](int tt, bf16 *Kn, bf16 *Vn) __attribute__((always_inline)) {
    const bool win = tt >= n_pref;
    const int64_t sp = win ? w_row : p_row;
    const int rowb = (int)(sp * 2);
    int base = tile_base(tt), limit = tile_limit(tt);
    const bf16 *kbase = win ? wkb : pkb, *vbase = win ? wvb : pvb;
    if (BT && !win) {
      // tile of keys [k0, k0 + 64) of the item's list: position k0 % page
      // of its page (pages hold multiples of 64 keys); a page id outside the
      // store contributes no rows
      const int k0 = base;
      const int pg = __builtin_amdgcn_readfirstlane(pg_next);
      const bool pok = pg >= 0 && pg < a.p_cap;
      const int64_t off = (int64_t)(pok ? pg : 0) * a.ps[0] + (int64_t)(k0 % a.page) * p_row;
      kbase = pkb + off - (int64_t)k0 * p_row;   // rsrc adds base * row again
      vbase = pvb + off - (int64_t)k0 * p_row;
      if (!pok) limit = base;
      const int rows = min(limit - base, kTK);
      if (tt & 1) rows_buf1 = rows;
      else rows_buf0 = rows;
    }
    // lane offset: row (lane / 16) of the block at the tile's row stride
    const int lrow = win ? lrow_w : lrow_p;
    if (stage_k) {
      const int wk = __builtin_amdgcn_readfirstlane(wave) - (S::SPLIT_STAGE ? 4 : 0);
      const auto r = rsrc(kbase, sp, base, limit);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int blk = wk * 4 + p;
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)&Kn[blk * 512], 16,
                                                 blk * 4 * rowb + lrow + kchunk[p], 0, 0, 0);
#else
        (void)r, (void)blk, (void)rowb, (void)lrow;   // the builtin exists in the device pass only
#endif
      }
    }
    if (stage_v) {
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      const auto r = rsrc(vbase, sp, base, limit);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int blk = wv * 4 + p;
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)&Vn[blk * 512], 16,
                                                 blk * 4 * rowb + lrow + vchunk, 0, 0, 0);
#else
        (void)r, (void)blk, (void)rowb, (void)lrow;
#endif
      }
    }
    request_page(tt + 1);
  };
  f32x16 acc[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY;  // reference max of scaled scores (log2 units)
  // this lane's share of the softmax denominator, in four partial sums.  It
  // sums the bf16-rounded weights the P V MFMAs use (bf16 dot products with
  // ones), so the weights applied to V sum to one.
  float l4[4] = {0.f, 0.f, 0.f, 0.f};
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};

  // ---- one tile: S^T = K Q^T, softmax, O^T += V^T P^T
  // fragment reads run kFragAhead MFMAs ahead of their use (rolling window,
  // fully unrolled; the order is pinned with sched_group_barrier, since the
  // scheduler otherwise moves each read next to its MFMA), so the LDS
  // latency is covered inside the wave.  3 to 5 measure the same; 6 is
  // slower.
  constexpr int kFragAhead = 4;
  auto kfrag = [&](const bf16 *Kb, int i) __attribute__((always_inline)) {  // K fragment i = ks * 2 + kt
    const int row = (i & 1) * 32 + ln, c = (i >> 1) * 2 + hh;
    return ld_bf16x8(&Kb[row * kKRow + ((c ^ (row & 15)) << 3)]);
  };
  // V^T fragment j = kt * 8 + k2 * 4 + dt from key-major V by two
  // transposing reads: lane (hh, ln) gets V[kb + hh*4 + e][db + ln] and
  // V[kb + 8 + hh*4 + e][db + ln] (e < 4), the keys its S^T accumulator
  // registers hold; chunk c of key row r sits at chunk c ^ 4 (r mod 4)
  const int tr_g = lane >> 4, tr_j = lane & 15;
  const int tr_row = (tr_g >> 1) * 4 + (tr_j >> 2);    // + kb (a multiple of 16)
  const int tr_col = 16 * (tr_g & 1) + 4 * (tr_j & 3);  // + db (a multiple of 32)
  auto vfrag = [&](const bf16 *Vb, int j) __attribute__((always_inline)) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef short v8s __attribute__((ext_vector_type(8)));
    const int kb = (j >> 3) * 32 + ((j >> 2) & 1) * 16, db = (j & 3) * 32;
    const int row = kb + tr_row, col = db + tr_col;
    const bf16 *p = &Vb[row * kD + (((col >> 3) ^ ((row & 3) << 2)) << 3) + (col & 7)];
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(p + 8 * kD));
    const v8s w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, w);
  };
  auto tile = [&](int tt, int buf, const bf16 *Kb, const bf16 *Vb) __attribute__((always_inline)) {
    f32x16 s[2];
    // the two 32-key halves interleaved: two independent accumulator chains
    s[0] = f32x16{};
    s[1] = f32x16{};
    bf16x8 kf[16];
#pragma unroll
    for (int i = 0; i < kFragAhead; ++i) kf[i] = kfrag(Kb, i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + kFragAhead < 16) kf[i + kFragAhead] = kfrag(Kb, i + kFragAhead);
      s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qop[i >> 1], s[i & 1], 0, 0, 0);
    }
    // the first V^T fragments are read while the softmax runs
    bf16x8 vf[16];
#pragma unroll
    for (int j = 0; j < kFragAhead; ++j) vf[j] = vfrag(Vb, j);
    // schedule: kFragAhead reads, then (1 MFMA, 1 read) x 16 (the last
    // kFragAhead reads are the V^T prefetches)
    __builtin_amdgcn_sched_group_barrier(0x100, kFragAhead, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    const int base = tile_base(tt);
    // keys of the tile past `limit` are not visible (block-table prefix
    // tiles: the rows their page holds)
    const int limit = (BT && tt < n_pref) ? base + (buf ? rows_buf1 : rows_buf0) : tile_limit(tt);
    const bool win = tt >= n_pref;
    if (win || base + kTK > limit) {
      // register r of half kt holds key base + kt*32 + (r/4)*8 + hh*4 + r%4;
      // the lane part goes into the threshold so the offsets are immediates
      const int thr = (win ? lim : limit) - base - hh * 4;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * 32 + (r >> 2) * 8 + (r & 3) >= thr) s[kt][r] = -INFINITY;
      if (WM && win) {
        const int lo_t = w_floor - base - hh * 4, sh_t = w_shared - base - hh * 4;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = kt * 32 + (r >> 2) * 8 + (r & 3);
            if (kk < lo_t && kk >= sh_t) s[kt][r] = -INFINITY;
          }
      }
    }
    // column max of the tile; the reference max is raised only when the
    // tile's max exceeds it by more than 2^8
    // (pairwise trees: short dependency chains between the S MFMAs and the
    // exponentials)
    // (three-input maxima: 32 -> 11 -> 4 -> 1)
    float m11[11], m4[4];
#pragma unroll
    for (int r = 0; r < 10; ++r) {
      const int e = 3 * r;
      m11[r] = fmaxf(fmaxf(s[e >> 4][e & 15], s[(e + 1) >> 4][(e + 1) & 15]), s[(e + 2) >> 4][(e + 2) & 15]);
    }
    m11[10] = fmaxf(s[1][14], s[1][15]);
#pragma unroll
    for (int r = 0; r < 3; ++r) m4[r] = fmaxf(fmaxf(m11[3 * r], m11[3 * r + 1]), m11[3 * r + 2]);
    m4[3] = fmaxf(m11[9], m11[10]);
    const float m1 = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    const float mx = fmaxf(m1, xor32(m1)) * a.scale2;
    const bool up = mx > m_run + kRescaleSlack;
    if (__ballot(up)) {
      const float m_new = up ? mx : m_run;
      const float alpha = up ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      m_run = m_new;
#pragma unroll
      for (int e = 0; e < 4; ++e) l4[e] *= alpha;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // p = exp2(score * scale2 - m); masked scores are -inf and give 0
      bf16x8 pop[2];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pop[r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], a.scale2, neg_m));
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x2x4 pp = __builtin_bit_cast(bf16x2x4, pop[k2]);
#pragma unroll
        for (int e = 0; e < 4; ++e) l4[e] = __builtin_amdgcn_fdot2_f32_bf16(pp.v[e], ones, l4[e], false);
      }
      // k-steps outer: four independent accumulators between dependent MFMAs
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) {
          const int j = kt * 8 + k2 * 4 + dt;
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], pop[k2], acc[dt], 0, 0, 0);
          if (j + kFragAhead < 16) vf[j + kFragAhead] = vfrag(Vb, j + kFragAhead);
          // MFMAs and LDS reads keep this order (read j+4 after MFMA j);
          // VALU, SALU and transcendental work may move across
          __builtin_amdgcn_sched_barrier(0x406);
        }
      }
    }
  };

  // ---- tile loop: tile tt+1 is loaded during tile tt (double-buffered LDS)
  request_page(0);
  if (n_tiles > 0) load(0, Ks0, Vt0);
  // every load issued so far (Q, tile 0) has landed: the loop below then
  // only waits for its own prefetches, at the LDS stores and the barrier
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // the K / V transfers into a buffer complete before the barrier that ends
  // the tile (an explicit wait on the vector memory counter, which counts
  // them: the barrier's own fence covers only what the compiler tracks), so
  // the next tile reads them after every wave's have landed
  auto step = [&](int tt, int buf, const bf16 *Kb, const bf16 *Vb, bf16 *Kn, bf16 *Vn)
      __attribute__((always_inline)) {
    if (tt + 1 < n_tiles) load(tt + 1, Kn, Vn);
    tile(tt, buf, Kb, Vb);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int tt = 0; tt < n_tiles; tt += 2) {
    step(tt, 0, Ks0, Vt0, Ks1, Vt1);
    if (tt + 1 < n_tiles) step(tt + 1, 1, Ks1, Vt1, Ks0, Vt0);
  }

  // ---- epilogue
  float l_run = (l4[0] + l4[1]) + (l4[2] + l4[3]);
  l_run += xor32(l_run);
  if (it.nc == 1) {
    if (!qok) return;
    const float inv = 1.f / l_run;
    bf16 *op = reinterpret_cast<bf16 *>(a.out) + (int64_t)b * a.os[0] + (int64_t)qi * a.os[1] +
               (int64_t)hq * a.os[2];
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[dt][rq * 4 + e] * inv);
        *reinterpret_cast<bf16x4 *>(op + dt * 32 + rq * 8 + hh * 4) = w;
      }
    }
    if (a.lse && hh == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.q + qi] = (m_run + __log2f(l_run)) * kLn2;
  } else {
    // partials [unit][chunk][column], unit = (natural row, KV head, query
    // tile).  The chunk's O / l (a convex combination of V rows, so within
    // V's range) is stored in bf16; (max, sum) stay fp32.  O of a 32-column
    // group is stored as [dims / 4][column][4]: lane l's store s (dims
    // 8s + 4hh ..) lands at element (64s + l) * 4, so each store instruction
    // writes 512 bytes contiguous.
    const int64_t unit = ((int64_t)it.rl * a.Hkv + h) * a.nqt + it.u;
    const int col = wave * 32 + ln;
    const int64_t prow = (unit * a.n_split + it.c) * S::NCOL + col;
    bf16 *po = a.part_o + (prow - ln) * kD + lane * 4;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(acc[dt][rq * 4 + e] * inv);
        *reinterpret_cast<bf16x4 *>(po + (dt * 4 + rq) * 256) = w;
      }
    if (hh == 0) {
      a.part_ml[prow * 2 + 0] = m_run;
      a.part_ml[prow * 2 + 1] = l_run;
    }
  }
}

// Merge the split-KV partials: one thread per (column, 4 dims), chunks in a
// fixed order, so the result does not depend on scheduling.  A block takes
// CPB columns (32: one column group, 1024 threads; 8 for the long chunk
// lists): CPB consecutive threads take its CPB columns of the same 4 dims,
// which in the partials' [dims / 4][column][4] order are 8 CPB contiguous
// bytes.  (Blocks of 8 columns for the short lists, four times as many,
// measured 4.6 % slower on the packed wavefronts: the launch is short and
// block dispatch counts.)
// U: partials requested per round of loads (8, or 32 for long chunk lists).
template <int NW, int G, int U, bool BT, int CPB>
__global__ __launch_bounds__(CPB * kD / 4) void attn_combine_kernel(AttnArgs a) {
  using S = Shape<NW, G>;
  const int blocks_per_unit = S::NCOL / CPB;
  const int64_t unit = blockIdx.x / blocks_per_unit;
  const int col = (blockIdx.x - unit * blocks_per_unit) * CPB + (threadIdx.x & (CPB - 1));
  const int d4 = threadIdx.x / CPB;
  const int u = (int)(unit % a.nqt);
  const int64_t group = unit / a.nqt;
  const int rl = (int)(group / a.Hkv);
  const int h = (int)(group - (int64_t)rl * a.Hkv);
  const int cg = col / 32;
  const int g = cg / S::QB;
  const int qb = cg - g * S::QB;
  const int qoff = u * S::NQ + qb * 32 + (col & 31);
  if (!BT && qoff >= a.q) return;
  const int64_t prow0 = unit * a.n_split * S::NCOL + col;
  // the partials of the first U chunks are requested before the row lookup
  // (row id, then prefix length), so the two latencies overlap; chunks past
  // the row's count hold stale data and are never used
  float2 ml[U];
  bf16x4 po[U];
  auto load = [&](int c0, int lim) {
#pragma unroll
    for (int v = 0; v < U; ++v) {
      if (c0 + v < lim) {
        const int64_t prow = prow0 + (int64_t)(c0 + v) * S::NCOL;
        ml[v] = *reinterpret_cast<const float2 *>(a.part_ml + prow * 2);
        po[v] = *reinterpret_cast<const bf16x4 *>(a.part_o + (prow - (col & 31)) * kD + (d4 * 32 + (col & 31)) * 4);
      }
    }
  };
  load(0, a.n_split);
  int b, P, qi;
  if constexpr (BT) {
    int q0, q1, toff;
    if (!bt_item(a, rl, b, q0, q1, toff, P)) return;
    qi = q0 + qoff;
    if (qi >= q1) return;
  } else {
    const RowRef rr = row_ref(a, rl);
    b = rr.b;
    if (b < 0 || b >= a.B) return;
    P = prefix_len(a, rr);
    qi = qoff;
  }
  const int nc = P > 0 ? (int)cdiv(P, a.chunk) : 1;
  if (nc == 1) return;  // written directly by the attention kernel
  // online merge in chunk order (every chunk holds visible prefix keys, so
  // each partial max is finite)
  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nc; c0 += U) {
    if (c0 > 0) load(c0, nc);
#pragma unroll
    for (int v = 0; v < U; ++v) {
      if (c0 + v < nc) {
        // the partial holds O / l: its weight is l * 2^(m - M)
        const float mn = fmaxf(M, ml[v].x);
        const float sa = __builtin_amdgcn_exp2f(M - mn);
        const float sb = ml[v].y * __builtin_amdgcn_exp2f(ml[v].x - mn);
        L = L * sa + sb;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = acc[e] * sa + (float)po[v][e] * sb;
        M = mn;
      }
    }
  }
  const float inv = 1.f / L;
  const int hq = h * G + g;
  bf16 *op = reinterpret_cast<bf16 *>(a.out) + (int64_t)b * a.os[0] + (int64_t)qi * a.os[1] +
             (int64_t)hq * a.os[2] + d4 * 4;
  bf16x4 w4;
#pragma unroll
  for (int e = 0; e < 4; ++e) w4[e] = (bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x4 *>(op) = w4;
  if (a.lse && d4 == 0) a.lse[((int64_t)b * a.Hq + hq) * a.q + qi] = (M + __log2f(L)) * kLn2;
}

// Rank the listed rows by prefix length, longest first (ties by list
// position), so that blocks start on the longest rows.  One block.
constexpr int kOrderMax = 1024;
__global__ __launch_bounds__(1024) void attn_order_kernel(AttnArgs a) {
  __shared__ int len[kOrderMax];
  const int n = a.n_rows;
  for (int r = threadIdx.x; r < n; r += blockDim.x) {
    const RowRef rr = row_ref(a, r);
    len[r] = (rr.b < 0 || rr.b >= a.B) ? -1 : prefix_len(a, rr);
  }
  __syncthreads();
  for (int r = threadIdx.x; r < n; r += blockDim.x) {
    const int lr = len[r];
    int rank = 0;
    for (int r2 = 0; r2 < n; ++r2) {
      const int l2 = len[r2];
      rank += (l2 > lr) || (l2 == lr && r2 < r);
    }
    a.row_order[rank] = r;
  }
}

// -------------------------------------------------------------- general path
// One block per (row, query head, 32-query tile); 8 lanes per query, each
// lane owning D/8 dimensions.  Keys are handled in batches of 8: each lane
// forms its partial dot products for the 8 keys (independent chains), the 8
// lanes add them (three butterfly steps per key, the 8 keys interleaved), and
// the running max and O are updated once per batch.  KG key groups of 256
// threads (launches with fewer blocks than CUs) take tiles kg, kg + KG, ...
// in lockstep with their own LDS buffers and hand (max, sum, O) to group 0
// through LDS at the end.  fp32 arithmetic throughout; used for fp32
// inputs and for shapes the MFMA path is not built for.
constexpr int kGenKeys = 32;
constexpr int kQT = 32;  // queries per block

template <typename T, int D, int KG>
__global__ __launch_bounds__(256 * KG) void attn_generic_kernel(AttnArgs a) {
  constexpr int DL = D / 8;  // dims per lane
  constexpr int EPT = kGenKeys * D / 256;  // tile elements staged per thread
  constexpr int KS = D + 4;  // LDS row stride (floats), 16-byte aligned rows
  __shared__ __attribute__((aligned(16))) float Kt[KG][2][kGenKeys][KS];
  __shared__ __attribute__((aligned(16))) float Vt_[KG][2][kGenKeys][KS];
  const int kg = KG > 1 ? (int)(threadIdx.x >> 8) : 0;  // key group
  const int tid = threadIdx.x & 255;
  const int ql = tid >> 3;   // query inside tile
  const int sub = tid & 7;   // dimension slice
  const int nqt = a.nqt;
  // block = (chunk, query tile, query head, row); chunk c covers prefix keys
  // [c * chunk, (c + 1) * chunk), the last chunk also the window
  const int64_t unit_id = blockIdx.x / a.n_split;
  const int c = (int)(blockIdx.x - unit_id * a.n_split);
  int unit = (int)unit_id;
  const int u = unit % nqt;
  unit /= nqt;
  const int hq = unit % a.Hq;
  const int rl = unit / a.Hq;
  const RowRef rr = row_ref(a, rl);
  const int b = rr.b;
  if (b < 0 || b >= a.B) return;
  const int h = hq / a.G;
  const int P_row = prefix_len(a, rr);
  const int nc = P_row > 0 ? (int)cdiv(P_row, a.chunk) : 1;
  if (c >= nc) return;
  const int kbeg = c * a.chunk;
  const int P = min(P_row, kbeg + a.chunk);   // end of this chunk's prefix keys
  const bool with_window = c == nc - 1;
  const int qi = u * kQT + ql;
  const bool q_ok = qi < a.q;
  const int ilast = min(u * kQT + kQT, a.q) - 1;
  const int win_len = window_limit(ilast, a.bl, a.q);
  const int lim_i = window_limit(q_ok ? qi : ilast, a.bl, a.q);
  const int w_floor = window_floor(q_ok ? qi : ilast, a.bl, a.mask_mode);
  const int w_shared = window_shared(a.bl, a.mask_mode);

  float qv[DL], o[DL];
  const T *qp = reinterpret_cast<const T *>(a.Q) + (int64_t)b * a.qs[0] + (int64_t)qi * a.qs[1] +
                (int64_t)hq * a.qs[2] + sub * DL;
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    qv[e] = q_ok ? (float)qp[e] : 0.f;
    o[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const PrefixSrc src = prefix_src(a, rr, h, (int)sizeof(T));
  const T *pkb = reinterpret_cast<const T *>(src.k);
  const T *pvb = reinterpret_cast<const T *>(src.v);
  const int64_t p_row = src.row;
  const T *wkb = reinterpret_cast<const T *>(a.wk) + (int64_t)b * a.ws[0] + (int64_t)h * a.ws[2];
  const T *wvb = reinterpret_cast<const T *>(a.wv) + (int64_t)b * a.ws[0] + (int64_t)h * a.ws[2];
  const int npt = (int)cdiv(P - kbeg, kGenKeys);
  const int nwt = with_window ? (int)cdiv(win_len, kGenKeys) : 0;
  const int ntile = npt + nwt;
  // staging: element tid + 256 i of the tile (consecutive threads on
  // consecutive dims), every load of a tile in flight together; tile t+1 is
  // loaded while tile t is computed (LDS double buffer)
  float kreg[EPT], vreg[EPT];
  auto gload = [&](int tile) {
    const bool win = tile >= npt;
    const int base = win ? (tile - npt) * kGenKeys : kbeg + tile * kGenKeys;
    const int limit = win ? win_len : P;
    const T *kb = win ? wkb : pkb;
    const T *vb = win ? wvb : pvb;
    const int64_t sp = win ? a.ws[1] : p_row;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + 256 * i;
      const int key = e / D, dd = e - key * D;
      const int gk = base + key;
      const bool ok = gk < limit;
      kreg[i] = ok ? (float)kb[(int64_t)gk * sp + dd] : 0.f;
      vreg[i] = ok ? (float)vb[(int64_t)gk * sp + dd] : 0.f;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + 256 * i;
      const int key = e / D, dd = e - key * D;
      Kt[kg][buf][key][dd] = kreg[i];
      Vt_[kg][buf][key][dd] = vreg[i];
    }
  };
  if (kg < ntile) {
    gload(kg);
    lstore(0);
  }
  __syncthreads();
  const int n_steps = (int)cdiv(ntile, KG);
  for (int step = 0; step < n_steps; ++step) {
    const int tile = step * KG + kg;
    const int buf = step & 1;
    const bool more = tile + KG < ntile;
    if (more) gload(tile + KG);
    if (tile < ntile) {
    const bool win = tile >= npt;
    const int base = win ? (tile - npt) * kGenKeys : kbeg + tile * kGenKeys;
    const int limit = win ? win_len : P;
    const int vlim = win ? lim_i : limit;   // keys at or past vlim are not visible
    // the tile in groups of 8 keys (a runtime loop bounds the registers the
    // scheduler can fill with LDS reads): scores of the group's keys, every
    // lane of the query holding all 8
#pragma unroll 1
    for (int k0 = 0; k0 < kGenKeys; k0 += 8) {
      float sc[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const float *kr = &Kt[kg][buf][k0 + kk][sub * DL];
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < DL; e += 4) {
          const f32x4 kv = *reinterpret_cast<const f32x4 *>(kr + e);
          dot = fmaf(qv[e + 0], kv[0], dot);
          dot = fmaf(qv[e + 1], kv[1], dot);
          dot = fmaf(qv[e + 2], kv[2], dot);
          dot = fmaf(qv[e + 3], kv[3], dot);
        }
        sc[kk] = dot;
      }
      float gmax = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        float dot = sc[kk];
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        dot += __shfl_xor(dot, 4);
        const int key = base + k0 + kk;
        bool vis = key < vlim;
        if (win && key < w_floor && key >= w_shared) vis = false;
        sc[kk] = vis ? dot * a.scale2 : -INFINITY;
        gmax = fmaxf(gmax, sc[kk]);
      }
      if (gmax > m_run) {
        // m_run = -inf gives alpha = 0 on an all-zero O and sum
        const float alpha = __builtin_amdgcn_exp2f(m_run - gmax);
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < DL; ++e) o[e] *= alpha;
        m_run = gmax;
      }
      const float mref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const float p = __builtin_amdgcn_exp2f(sc[kk] - mref);
        l_run += p;
        const float *vr = &Vt_[kg][buf][k0 + kk][sub * DL];
#pragma unroll
        for (int e = 0; e < DL; e += 4) {
          const f32x4 vv = *reinterpret_cast<const f32x4 *>(vr + e);
          o[e + 0] = fmaf(p, vv[0], o[e + 0]);
          o[e + 1] = fmaf(p, vv[1], o[e + 1]);
          o[e + 2] = fmaf(p, vv[2], o[e + 2]);
          o[e + 3] = fmaf(p, vv[3], o[e + 3]);
        }
      }
    }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }
  if constexpr (KG > 1) {
    // groups 1.. -> LDS as [group - 1][value][thread] (the tile buffers are
    // free after the loop's last barrier); group 0 merges them in group order
    float *xg = &Kt[0][0][0][0];
    static_assert((KG - 1) * (DL + 2) * 256 <= KG * 2 * kGenKeys * KS, "hand-over area exceeds the K tiles");
    if (kg > 0) {
      float *x = xg + (kg - 1) * (DL + 2) * 256 + tid;
      x[0] = m_run;
      x[256] = l_run;
#pragma unroll
      for (int e = 0; e < DL; ++e) x[(2 + e) * 256] = o[e];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int g = 1; g < KG; ++g) {
      const float *x = xg + (g - 1) * (DL + 2) * 256 + tid;
      const float mg = x[0];
      const float mm = fmaxf(m_run, mg);
      // a group with no visible key has max -inf, sum 0 and O 0: weight 0
      const float w0 = m_run == mm ? 1.f : __builtin_amdgcn_exp2f(m_run - mm);
      const float w1 = mg == mm ? 1.f : __builtin_amdgcn_exp2f(mg - mm);
      l_run = l_run * w0 + x[256] * w1;
#pragma unroll
      for (int e = 0; e < DL; ++e) o[e] = o[e] * w0 + x[(2 + e) * 256] * w1;
      m_run = mm;
    }
  }
  if (!q_ok) return;
  const float inv = 1.f / l_run;
  if (nc > 1) {
    // partial of chunk c: O / l in fp32 and (max, sum); rows [unit][chunk][query]
    const int64_t prow = (unit_id * a.n_split + c) * kQT + ql;
    float *po = a.gpart_o + prow * D + sub * DL;
#pragma unroll
    for (int e = 0; e < DL; e += 4)
      *reinterpret_cast<f32x4 *>(po + e) = f32x4{o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
    if (sub == 0) *reinterpret_cast<float2 *>(a.part_ml + prow * 2) = float2{m_run, l_run};
    return;
  }
  T *op = reinterpret_cast<T *>(a.out) + (int64_t)b * a.os[0] + (int64_t)qi * a.os[1] +
          (int64_t)hq * a.os[2] + sub * DL;
#pragma unroll
  for (int e = 0; e < DL; ++e) op[e] = (T)(o[e] * inv);
  if (a.lse && sub == 0) a.lse[((int64_t)b * a.Hq + hq) * a.q + qi] = (m_run + log2f(l_run)) * kLn2;
}

// Merge the general path's split partials: one thread per (query, 4 dims)
// of a (row, query head, query tile) unit, chunks in a fixed order.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_generic_combine_kernel(AttnArgs a) {
  constexpr int D4 = D / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int d4 = (int)(idx % D4);
  const int64_t r = idx / D4;
  const int ql = (int)(r % kQT);
  const int64_t unit_id = r / kQT;
  int unit = (int)unit_id;
  const int u = unit % a.nqt;
  unit /= a.nqt;
  const int hq = unit % a.Hq;
  const int rl = unit / a.Hq;
  if (rl >= a.n_rows) return;
  const RowRef rr = row_ref(a, rl);
  const int b = rr.b;
  if (b < 0 || b >= a.B) return;
  const int qi = u * kQT + ql;
  if (qi >= a.q) return;
  const int P = prefix_len(a, rr);
  const int nc = P > 0 ? (int)cdiv(P, a.chunk) : 1;
  if (nc == 1) return;   // written directly by the attention kernel
  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int cc = 0; cc < nc; ++cc) {
    const int64_t prow = (unit_id * a.n_split + cc) * kQT + ql;
    const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + prow * 2);
    const f32x4 po = *reinterpret_cast<const f32x4 *>(a.gpart_o + prow * D + d4 * 4);
    // every chunk holds visible prefix keys: each partial max is finite
    const float mn = fmaxf(M, ml.x);
    const float sa = __builtin_amdgcn_exp2f(M - mn);
    const float sb = ml.y * __builtin_amdgcn_exp2f(ml.x - mn);
    L = L * sa + sb;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = acc[e] * sa + po[e] * sb;
    M = mn;
  }
  const float inv = 1.f / L;
  T *op = reinterpret_cast<T *>(a.out) + (int64_t)b * a.os[0] + (int64_t)qi * a.os[1] +
          (int64_t)hq * a.os[2] + d4 * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) op[e] = (T)(acc[e] * inv);
  if (a.lse && d4 == 0) a.lse[((int64_t)b * a.Hq + hq) * a.q + qi] = (M + log2f(L)) * kLn2;
}

}  // namespace

bool attn_mfma_supported(int dtype, int d, int G) {
  return dtype == BD_BF16 && d == kD && (G == 1 || G == 2 || G == 4 || G == 8);
}

bool attn_generic_supported(int dtype, int d) {
  return (dtype == BD_BF16 || dtype == BD_F32) && (d == 64 || d == 128);
}

// Plan of the MFMA path.  Blocks of 4 waves serve GQA groups of at most 4
// when one query tile of 4 waves covers every query (q * G <= 128);
// otherwise 8 waves.  The prefix is cut into chunks only while there are
// fewer blocks than block slots on the GPU (one 8-wave or two 4-wave blocks
// per CU), and
// never below kMinChunk keys: each extra chunk costs a partial O row of
// 256 bytes per column.  Rows are ordered longest first when the blocks do
// not all fit at once.
constexpr int kCUs = 256;
constexpr int kMinChunk = 256;

AttnPlan attn_plan(int dtype, int B, int Hq, int Hkv, int d, int q, int n_rows, int p_max,
                   bool keep_order) {
  (void)B;
  AttnPlan p{};
  const int G = Hkv > 0 ? Hq / Hkv : 1;
  p.chunk = 1 << 30;
  p.n_split = 1;
  if (!attn_mfma_supported(dtype, d, G)) {
    // general path: blocks of one (row, query head, 32-query tile); with
    // fewer blocks than CUs the prefix is cut into chunks of whole 32-key
    // tiles (one tile at least), each writing an fp32 O / l with its
    // (max, sum), merged by a combine kernel in chunk order
    p.nw = 0;
    p.nqt = (int)cdiv(q, kQT);
    const int64_t units = (int64_t)n_rows * Hq * p.nqt;
    if (p_max > kGenKeys && units < kCUs) {
      const int64_t want = cdiv(kCUs, units);
      const int64_t ch = cdiv(cdiv(p_max, want), kGenKeys) * kGenKeys;
      if (ch < p_max) {
        p.chunk = (int)ch;
        p.n_split = (int)cdiv(p_max, ch);
        const size_t prows = (size_t)units * p.n_split * kQT;
        p.off_part_o = 0;
        p.off_part_ml = align256(prows * d * sizeof(float));
        p.ws_bytes = p.off_part_ml + align256(prows * 2 * sizeof(float));
      }
    }
    return p;
  }
  p.nw = ((int64_t)q * G <= 128 && G <= 4) ? 4 : 8;
  const int ncg = p.nw;
  const int nq = 32 * (ncg / G);
  const int ncol = 32 * ncg;
  p.nqt = (int)cdiv(q, nq);
  const int64_t slots = (int64_t)kCUs * (p.nw == 4 ? 2 : 1);
  const int64_t units = (int64_t)n_rows * Hkv * p.nqt;
  if (p_max > 0 && units < slots) {
    const int64_t want = cdiv(slots, units);
    int64_t ch = cdiv(cdiv(p_max, want), kTK) * kTK;
    if (ch < kMinChunk) ch = kMinChunk;
    if (ch < p_max) {
      p.chunk = (int)ch;
      p.n_split = (int)cdiv(p_max, ch);
    }
  }
  p.order = !keep_order && n_rows > 1 && n_rows <= kOrderMax && units * p.n_split > slots;
  size_t off = 0;
  p.off_order = off;
  if (p.order) off += align256((size_t)n_rows * sizeof(int));
  p.off_part_o = off;
  p.off_part_ml = off;
  if (p.n_split > 1) {
    const size_t prows = (size_t)units * p.n_split * ncol;
    off += align256(prows * kD * sizeof(bf16));
    p.off_part_ml = off;
    off += align256(prows * 2 * sizeof(float));
  }
  p.ws_bytes = off;
  return p;
}

template <int NW, int G>
static hipError_t launch_mfma(const AttnArgs &a, hipStream_t s) {
  const bool wm = a.mask_mode != BD_MASK_BLOCK_CAUSAL;
  const bool bt = a.items != nullptr;
  using S = Shape<NW, G>;
  const int64_t n_groups = (int64_t)a.n_rows * a.Hkv;
  const int64_t per_group = (int64_t)a.nqt * a.n_split;
  const int64_t grid = 8 * cdiv(n_groups, 8) * per_group;
  if (a.row_order) {
    hipLaunchKernelGGL(attn_order_kernel, dim3(1), dim3(kOrderMax), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (bt)
    hipLaunchKernelGGL((attn_mfma_kernel<NW, G, false, true>), dim3((unsigned)grid), dim3(S::NT), 0, s, a);
  else if (wm)
    hipLaunchKernelGGL((attn_mfma_kernel<NW, G, true, false>), dim3((unsigned)grid), dim3(S::NT), 0, s, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<NW, G, false, false>), dim3((unsigned)grid), dim3(S::NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split <= 1) return e;
  // one round of loads covers up to 8 chunks, in blocks of 32 columns; longer
  // lists (pools of thousands of keys) take 32 per round, fewer dependent
  // round trips, in blocks of 8 columns (their 32 partials in flight per
  // thread need more registers than a 1024-thread block leaves)
  const int64_t cgrid8 = n_groups * a.nqt * (S::NCOL / 8), cgrid32 = n_groups * a.nqt * (S::NCOL / 32);
  if (bt) {
    if (a.n_split > 8)
      hipLaunchKernelGGL((attn_combine_kernel<NW, G, 32, true, 8>), dim3((unsigned)cgrid8), dim3(8 * kD / 4), 0, s, a);
    else
      hipLaunchKernelGGL((attn_combine_kernel<NW, G, 8, true, 32>), dim3((unsigned)cgrid32), dim3(32 * kD / 4), 0, s, a);
  } else if (a.n_split > 8) {
    hipLaunchKernelGGL((attn_combine_kernel<NW, G, 32, false, 8>), dim3((unsigned)cgrid8), dim3(8 * kD / 4), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_combine_kernel<NW, G, 8, false, 32>), dim3((unsigned)cgrid32), dim3(32 * kD / 4), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a, hipStream_t s) {
  if (attn_mfma_supported(a.dtype, a.d, a.G)) {
    if (a.nw == 4) {
      switch (a.G) {
        case 1: return launch_mfma<4, 1>(a, s);
        case 2: return launch_mfma<4, 2>(a, s);
        case 4: return launch_mfma<4, 4>(a, s);
      }
    } else {
      switch (a.G) {
        case 1: return launch_mfma<8, 1>(a, s);
        case 2: return launch_mfma<8, 2>(a, s);
        case 4: return launch_mfma<8, 4>(a, s);
        case 8: return launch_mfma<8, 8>(a, s);
      }
    }
    return hipErrorInvalidValue;
  }
  const int64_t units = (int64_t)a.n_rows * a.Hq * a.nqt;
  const int64_t grid = units * a.n_split;
  // fewer blocks than CUs (a prefix too short to split): key groups per
  // block (4 at d = 64, 2 at d = 128, as the LDS allows)
  const bool few = grid < kCUs && a.n_split == 1;
  const dim3 g((unsigned)grid);
  if (a.dtype == BD_F32) {
    if (a.d == 64) {
      if (few) hipLaunchKernelGGL((attn_generic_kernel<float, 64, 4>), g, dim3(1024), 0, s, a);
      else hipLaunchKernelGGL((attn_generic_kernel<float, 64, 1>), g, dim3(256), 0, s, a);
    } else {
      if (few) hipLaunchKernelGGL((attn_generic_kernel<float, 128, 2>), g, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((attn_generic_kernel<float, 128, 1>), g, dim3(256), 0, s, a);
    }
  } else {
    if (a.d == 64) {
      if (few) hipLaunchKernelGGL((attn_generic_kernel<bf16, 64, 4>), g, dim3(1024), 0, s, a);
      else hipLaunchKernelGGL((attn_generic_kernel<bf16, 64, 1>), g, dim3(256), 0, s, a);
    } else {
      if (few) hipLaunchKernelGGL((attn_generic_kernel<bf16, 128, 2>), g, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((attn_generic_kernel<bf16, 128, 1>), g, dim3(256), 0, s, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split <= 1) return e;
  const dim3 cg((unsigned)cdiv(units * kQT * (a.d / 4), 256));
  if (a.dtype == BD_F32) {
    if (a.d == 64) hipLaunchKernelGGL((attn_generic_combine_kernel<float, 64>), cg, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_generic_combine_kernel<float, 128>), cg, dim3(256), 0, s, a);
  } else {
    if (a.d == 64) hipLaunchKernelGGL((attn_generic_combine_kernel<bf16, 64>), cg, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attn_generic_combine_kernel<bf16, 128>), cg, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bd
