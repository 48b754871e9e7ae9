// Prefix split-KV attention for DDTree verify over an MLA latent pool (gfx950).
//
// Every tree node attends densely to the whole prefix with no mask ("The
// Architecture Detective: Uncovering FlashMLA's Potential for Blackwell DDTree
// Verification", "The Message in Full": causal=False over the prefix, one
// latent head of width 576 whose first 512 columns are V).  The prefix is cut
// into fixed chunks of logical positions; each chunk yields a normalised
// partial (o_s, lse_s) that a later pass merges by log-sum-exp ("The Anatomy of
// a Kernel Investigation", "The Reasoning Process: A Deep Dive", Phase 2).
//
// Work item = (request b, row tile of 64 query rows, chunk s); one 256-thread
// workgroup (4 waves) per item.  All H*N query rows of a request read every
// prefix key, so the pass is a dense contraction and runs on MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Waves form two pairs; pair p owns query rows [32p, 32p+32) of the tile and
// wave (p, h) of the pair key block h (keys [32h, 32h+32) of each tile) and
// output columns [256h, 256h+256):
//   * QK: holds all 576 query columns of the pair's rows in VGPRs and computes
//     the scores S^T = K Q^T of its key block (A = K from LDS, B = Q).  In the
//     32x32 accumulator layout each lane owns one query row.
//   * softmax: P = exp2(S*scale*log2e - m) in bf16 for those 32 keys, also
//     stored to LDS for the partner (it is the partner's MFMA operand too).
//   * PV: O^T += V^T P^T for its 256 output columns over all 64 keys (A = V^T
//     read from the same LDS tile by ds_read_b64_tr_b16, B = P): first over
//     its own key block, then, after the tile's one barrier, over the
//     partner's with the P the partner stored.
// Per wave: Q 144 VGPRs and a 32x256 fp32 accumulator (128 AGPRs).  Splitting
// the pair by keys rather than by query columns leaves no partial scores to
// exchange, so a tile needs one barrier besides the one that hands over the
// staged tile.
//
// Gather: buffer_load_dwordx4 ... lds moves 16 bytes per lane straight into
// LDS (no VGPR staging).  Latent rows use the buffer (MUBUF) form with one
// descriptor per row, rope rows the global form issued through asm (see
// dma16_global): the compiler counts a global LDS-DMA as a pending LDS access
// until it completes, which would turn every LDS operand wait of the tile
// into a full drain; a buffer DMA is tracked as a plain vector-memory op.  Per key, one instruction fetches the 1 KB latent part of
// its pool row (8 cache lines); one instruction fetches the 128-byte rope parts
// of 8 keys.  Slots are held one per lane and loaded two tiles ahead.  LDS tile
// layout (72 KB per 64 keys):
//   latent: key k at k*1024, 16-byte piece c at slot c ^ g(k),
//           g(k) = ((k & 3) << 2) | ((k >> 2) & 3)
//   rope:   key k at 64 KB + k*128, piece c at slot c ^ ((k >> 1) & 7)
// Lane-linear DMA writes pick the piece each lane loads, so the swizzle is
// free; it keeps the ds_read_b128 (QK, 16 lanes per LDS cycle) and
// ds_read_b64_tr_b16 (PV, 32 lanes per cycle) patterns free of bank
// conflicts.  Tiles are double-buffered: the 18 gather instructions of tile
// t+1 are spread over the QK loop of tile t.
//
// Softmax reference: each row keeps a reference m (log2 units) instead of a
// running max, so the accumulator is never rescaled and stays in AGPRs.  The
// first tile sets m to the pair's tile max.  While every score stays within
// kSlack of m, exp2(s - m) <= 2^kSlack, far inside bf16/fp32 range.  A tile
// that breaks this (rare) makes the whole workgroup restart its chunk with
// m raised to that tile's max plus kSlack of headroom; m only grows, by more
// than kSlack per restart, so restarts are few and the result is the same.

#include "kernels.h"

namespace vamla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kSlack = 16.0f;     // scores may exceed the reference by this much (log2 units)
constexpr int kRopeBase = 64 * 1024;
constexpr int kPreQK = 4;           // LDS operand reads in flight ahead of their MFMA (QK)
constexpr int kPrePV = 4;           // same for PV (two transposed reads each)
constexpr int kQkSteps = kDqk / 16; // 36 MFMA steps over the query columns

// Which gather instruction of the next tile (0..17, or -1 for none) rides
// along with MFMA step g of a tile (QK steps 0..35, then PV steps 36..67; the
// PV loop offers steps 36 + 8ks + 4 + c, ks, c in 0..3).  The two rope
// instructions go first, the 16 latent ones with the PV steps, where the MFMA
// pipe rather than the LDS limits the wave.
__device__ __forceinline__ constexpr int dma_at(int g) {
  return g < 2 ? 16 + g : ((g >= 40 && ((g - 40) & 4) == 0) ? ((g - 40) >> 3) * 4 + ((g - 40) & 3) : -1);
}
// Buffer descriptor word 3 for plain dword loads (32-bit data format, no swizzle)
constexpr int kRsrcWord3 = 0x00020000;

// Exchange area, 48 bytes per lane and wave: wave w stores the P operand of
// its key block in v[w][0..1] and its row max and restart vote in v[w][2].
struct __attribute__((aligned(16))) Xchg {
  float4 v[4][3][64];               // [wave][16-byte part][lane], 12 KB
};

__device__ __forceinline__ int swz_latent(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }
__device__ __forceinline__ int swz_rope(int k) { return (k >> 1) & 7; }

// Workgroup barrier that waits only for this wave's LDS operations.  A fence
// would also wait for the in-flight gathers (LDS DMA counts as LDS stores),
// which must keep running under the math.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// base ^ c, computed where it is used (an opaque xor keeps the compiler from
// hoisting every variant of a swizzled base into its own register)
__device__ __forceinline__ int xor_at_use(int base, int c) {
  if (c == 0) return base;
  int r;
  asm volatile("v_xor_b32 %0, %2, %1" : "=v"(r) : "v"(base), "i"(c));   // literal must be src0
  return r;
}

__device__ __forceinline__ bf16x8 tr_pair(const uint8_t* base, int off1, int off2) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off1));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off2));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// LDS DMA of 16 bytes per lane from a 64-bit per-lane address into LDS at
// lds_addr + 16*lane (the rope parts of 8 keys from 8 unrelated rows; buffer
// offsets are 32-bit, so rows past 4 GiB of the pool need this form).  Written
// as asm so that the compiler's wait tracking does not see it: it would count
// the op as a pending LDS access until it completes and drain every LDS wait
// behind it.  The data is read only after the s_waitcnt 0 and barrier that
// start the next tile.  M0 carries the LDS address and is restored.
__device__ __forceinline__ void dma16_global(const void* src, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
}

// Pool slots of one wave's 16 keys of a tile, one per lane: `lat` holds the
// slot of key 16w + (lane & 15), rope[j] that of key 16w + 8j + (lane >> 3).
struct TileSlots {
  uint32_t lat, rope[2];
};

// Gather instruction d (0..17) of this wave's share of one key tile, keys
// [16w, 16w+16): d < 16 moves the 1 KB latent part of key 16w+d (one 64-lane
// instruction, 8 cache lines; the slot is read out of lane d), d = 16, 17 the
// 128-byte rope parts of keys 16w + 8(d-16) + (lane >> 3) (8 keys per 64-lane
// instruction).  Lanes write 16 bytes each, lane-linearly, and load the piece
// the swizzle puts there.
__device__ __forceinline__ void gather_one(const uint16_t* pool, const TileSlots& sl, uint8_t* lds, int w, int lane,
                                           int d) {
  if (d < 16) {
    const uint32_t slot = __builtin_amdgcn_readlane(sl.lat, d);
    const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc((void*)(pool + (size_t)slot * kDqk), 0, 1024,
                                                                         kRsrcWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(row, (lds_void*)(lds + (16 * w + d) * 1024), 16,
                                             (uint32_t)xor_at_use(lane << 4, swz_latent(d) << 4), 0, 0, 0);
  } else {
    const int j = d - 16;
    const int kl = 8 * j + (lane >> 3);                      // key within the wave's 16
    const uint8_t* src = (const uint8_t*)(pool + (size_t)sl.rope[j] * kDqk + 512) + (((lane & 7) ^ swz_rope(kl)) << 4);
    dma16_global(src, (uint32_t)(uintptr_t)(lds_void*)(lds + kRopeBase + (16 * w + 8 * j) * 128));
  }
}

__device__ __forceinline__ void gather_tile(const uint16_t* pool, const TileSlots& sl, uint8_t* lds, int w,
                                            int lane) {
#pragma unroll
  for (int d = 0; d < 18; ++d) gather_one(pool, sl, lds, w, lane, d);
}

struct Lane {
  int w, pr, hf, hl, l32, lane;
  // Swizzled LDS addresses are written base ^ (step-dependent bits) + immediate:
  // key = 32*hf + l32 (the lane's key of the wave's block)
  int qk_lat;        // latent: key*1024 | ((hl ^ g(key)) << 4); step s: ^ 32*(s&7), + 256*(s>>3)
  int qk_rope;       // rope: 64K + key*128 | ((hl ^ h(key)) << 4); rope step r: ^ 32*r
  int pv[2];         // PV transposed reads, key group sec: column block c: ^ 64*c
};

struct RowState {
  float m;   // reference max of scaled scores (log2 units), shared by the pair
  float l;   // this lane's share of the row sum
};

// K fragment of QK step s (0..35) of this wave's key block: 16-byte pieces
// 2s and 2s+1 of the 576 columns (latent for s < 32, then rope); lane half
// hl takes piece 2s + hl.
__device__ __forceinline__ bf16x8 kfrag(const uint8_t* lds, const Lane& ln, int s) {
  if (s < 32) return *(const bf16x8*)(lds + xor_at_use(ln.qk_lat, 32 * (s & 7)) + (s >> 3) * 256);
  return *(const bf16x8*)(lds + xor_at_use(ln.qk_rope, 32 * (s - 32)));
}

// x[lane] and x[lane ^ 32] for every lane, through one v_permlane32_swap of
// two copies of x (afterwards each lane holds one of the two values in each
// register).  Written as asm: handed the same value twice, the builtin's two
// results get folded into one.
__device__ __forceinline__ void halves32(float x, float& p, float& q) {
  p = x;
  q = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(p), "+v"(q));
}
__device__ __forceinline__ float max_xor32(float x) {
  float p, q;
  halves32(x, p, q);
  return fmaxf(p, q);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float p, q;
  halves32(x, p, q);
  return p + q;
}

// P = exp2(s*scale - m) in bf16 for this lane's 16 raw scores; lsum += sum P
// (four partial sums, so the adds do not form one long dependency chain).
__device__ __forceinline__ void pack_p(const f32x16& v, float scale, float m, bf16x8 (&pb)[2], float& lsum) {
  float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(v[half * 8 + e], scale, -m));
      part[e & 3] += p;
      pb[half][e] = (__bf16)p;
    }
  }
  lsum += (part[0] + part[1]) + (part[2] + part[3]);
}

// One staged 64-key tile for this wave.  `first` (workgroup-uniform): the
// chunk's reference m is not set yet.  Returns true when the workgroup must
// restart its chunk; the tile's contribution is then discarded.
__device__ __forceinline__ bool tile_math(const uint8_t* lds, Xchg& x, const bf16x8 (&qf)[kQkSteps],
                                          f32x16 (&o)[8], RowState& st, bool first, int nvalid, bool masked,
                                          uint64_t vis, float scale_log2,
                                          const Lane& ln, const uint16_t* pool, const TileSlots& ng_sl,
                                          uint8_t* ng_lds) {
  // S^T of this wave's key block over all 576 columns (a chain of dependent
  // MFMAs on one accumulator issues at full rate)
  f32x16 v = {};
  {
    bf16x8 kf[kPreQK];
#pragma unroll
    for (int i = 0; i < kPreQK; ++i) kf[i] = kfrag(lds, ln, i);
#pragma unroll
    for (int i = 0; i < kQkSteps; ++i) {
      const bf16x8 cur = kf[i % kPreQK];
      if (i + kPreQK < kQkSteps) kf[i % kPreQK] = kfrag(lds, ln, i + kPreQK);
      v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[i], v, 0, 0, 0);
      // on a chunk's last tile the gather refetches valid rows into the idle buffer
      if (dma_at(i) >= 0) gather_one(pool, ng_sl, ng_lds, ln.w, ln.lane, dma_at(i));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // lane holds keys 32*hf + 8*(r/4) + 4*hl + r%4 of row l32 (raw scores)
  if (nvalid < kKeyTile) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * ln.hf + 8 * (r >> 2) + 4 * ln.hl + (r & 3) >= nvalid) v[r] = -INFINITY;
  }
  if (masked) {       // tree keys: bit k of vis = key k of the tile is visible to this row
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (((vis >> (32 * ln.hf + 8 * (r >> 2) + 4 * ln.hl + (r & 3))) & 1) == 0) v[r] = -INFINITY;
  }
  float mt = v[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, v[r]);
  mt = max_xor32(mt) * scale_log2;                 // row max over the block's 32 keys, log2 units
  if (first) {
    // the reference is the pair's max over this tile
    x.v[ln.w][2][ln.lane] = make_float4(mt, 0.f, 0.f, 0.f);
    lds_barrier();
    st.m = fmaxf(mt, x.v[ln.w ^ 1][2][ln.lane].x);
  }
  bf16x8 pb[2];
  float lsum = 0.f;
  pack_p(v, scale_log2, st.m, pb, lsum);
  const float want = __any(mt > st.m + kSlack) ? 1.f : 0.f;   // never on the first tile
  x.v[ln.w][0][ln.lane] = __builtin_bit_cast(float4, pb[0]);
  x.v[ln.w][1][ln.lane] = __builtin_bit_cast(float4, pb[1]);
  x.v[ln.w][2][ln.lane] = make_float4(mt, want, 0.f, 0.f);
  // O^T += V^T P^T for this wave's 128 output columns [128w, 128w+128) over
  // all 64 rows and all 64 keys.  P of the four (row block, key block) pairs
  // comes from the four waves: this wave's from registers, the rest from LDS
  // behind the tile's barrier.  Each V^T fragment (32 columns x 16 keys) feeds
  // the MFMAs of both row blocks.  P keeps the key order of the score
  // accumulator layout and the transposed V reads take the keys in that same
  // order.  Key steps ks = 2*kb' + h run over the own key block (kb' = 0)
  // first; o[4*rb' + c] accumulates column block c of row block rb' (rb' = 0:
  // this pair's rows).
  {
    const int own0 = ln.pv[0] + ln.hf * 32768, own1 = ln.pv[1] + ln.hf * 32768;
    const int oth0 = own0 ^ 32768, oth1 = own1 ^ 32768;
    auto vfrag = [&](int ks, int c) {
      const int off = (ks & 1) * 16 * 1024;
      const int b0 = ks < 2 ? own0 : oth0, b1 = ks < 2 ? own1 : oth1;
      return tr_pair(lds, xor_at_use(b0, 64 * c) + off, xor_at_use(b1, 64 * c) + off);
    };
    bf16x8 vf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vf[c] = vfrag(0, c);
    lds_barrier();
    // P operands of the other waves, read as the key steps reach them:
    // (this pair's rows, other key block) from w^1, (other rows, own block)
    // from w^2, (other rows, other block) from w^3
    auto pfrom = [&](int wv, int h) { return __builtin_bit_cast(bf16x8, x.v[wv][h][ln.lane]); };
    bf16x8 q0n = pb[0], q1n = pfrom(ln.w ^ 2, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 q0 = q0n;                           // this pair's rows
      const bf16x8 q1 = q1n;                           // the other pair's rows
      if (ks < 3) {
        const int n = ks + 1, h = n & 1;
        q0n = n < 2 ? pb[h] : pfrom(ln.w ^ 1, h);
        q1n = pfrom(n < 2 ? ln.w ^ 2 : ln.w ^ 3, h);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c], q0, o[c], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        o[4 + c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c], q1, o[4 + c], 0, 0, 0);
        if (ks < 3) vf[c] = vfrag(ks + 1, c);
        if (dma_at(36 + 8 * ks + 4 + c) >= 0) gather_one(pool, ng_sl, ng_lds, ln.w, ln.lane, dma_at(36 + 8 * ks + 4 + c));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // The restart vote is read only now: a restarting chunk discards this
  // tile's accumulation anyway.  Every wave stored its wave-uniform vote in
  // all lanes, so each lane reads its own.
  const float any_flag = x.v[0][2][ln.lane].y + x.v[1][2][ln.lane].y + x.v[2][2][ln.lane].y + x.v[3][2][ln.lane].y;
  if (__builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, any_flag)) != 0) {
    // a score ran past the reference: restart the chunk with headroom
    const float mp = fmaxf(mt, x.v[ln.w ^ 1][2][ln.lane].x);
    st.m = fmaxf(st.m, mp) + kSlack;
    st.l = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = f32x16{};
    return true;
  }
  st.l += lsum;
  return false;
}

__global__ __launch_bounds__(256, 1) void prefix_splitkv_kernel(PrefixArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kTileBytes];
  __shared__ Xchg x;
  __shared__ int par_s[kMaxTree];                 // the request's parent array
  __shared__ uint64_t vis_s[kRowTile][2];         // per row: visible tree keys 0..63, 64..127

  Lane ln;
  ln.lane = threadIdx.x & 63;
  ln.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  ln.pr = ln.w >> 1;
  ln.hf = ln.w & 1;
  ln.hl = ln.lane >> 5;
  ln.l32 = ln.lane & 31;

  // Work item; consecutive logical items (the row tiles of one chunk) land on
  // one XCD, since workgroup i is dispatched to XCD i % 8.
  const int per_xcd = a.grid_items >> 3;
  const int k = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int tiles_chunks = a.row_tiles * a.max_chunks;
  if (k >= a.batch * tiles_chunks) return;
  const int b = k / tiles_chunks;
  const int rem = k - b * tiles_chunks;
  const int s = rem / a.row_tiles;
  const int tile = rem - s * a.row_tiles;
  const int p0 = a.cu_prefix[b];
  const int L = a.cu_prefix[b + 1] - p0;
  // chunks of this request; with no prefix, chunk 0 still carries the tree
  const int nchunks = max(1, min((L + a.chunk - 1) / a.chunk, a.max_chunks));
  if (s >= nchunks) return;
  const int kbeg = s * a.chunk;
  const int kend = min(kbeg + a.chunk, L);
  const int t0 = a.cu_tree[b];
  const int n_b = a.cu_tree[b + 1] - t0;
  const int rows_b = n_b * a.num_heads;
  if (tile * kRowTile >= rows_b) return;
  // The request's last chunk also takes its tree keys (<= 65, so at most two
  // tiles) under the ancestor-or-self mask ("Mapping the Optimization
  // Landscape for DDTree Verify Attention", "Input Knowledge Required to
  // Understand This Message", item 1): one partial then covers both.
  const int ntp = kend > kbeg ? (kend - kbeg + kKeyTile - 1) / kKeyTile : 0;   // prefix tiles
  const int ntt = s == nchunks - 1 ? (min(n_b, kMaxTree) + kKeyTile - 1) / kKeyTile : 0;   // tree tiles

  const int row_in_tile = ln.pr * 32 + ln.l32;
  const int row = tile * kRowTile + row_in_tile;
  const bool row_ok = row < rows_b;

  // the pair's query rows, all 576 columns: lane (l32, hl) holds 16-byte
  // piece 2s + hl of its row for step s (latent pieces 0..63, rope 64..71)
  bf16x8 qf[kQkSteps];
  {
    const uint16_t* qrow = a.q + ((size_t)t0 * a.num_heads + (row_ok ? row : 0)) * kDqk;
#pragma unroll
    for (int s2 = 0; s2 < kQkSteps; ++s2) {
      const int piece = 2 * s2 + ln.hl;
      bf16x8 v = *(const bf16x8*)(qrow + piece * 8);
      qf[s2] = row_ok ? v : bf16x8{};
    }
  }

  f32x16 o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x16{};
  RowState st{-INFINITY, 0.f};

  // lane constants for LDS reads (layout in the header comment)
  {
    const int key = 32 * ln.hf + ln.l32;
    ln.qk_lat = (key * 1024) | ((ln.hl ^ swz_latent(key)) << 4);
    ln.qk_rope = (kRopeBase + key * 128) | ((ln.hl ^ swz_rope(key)) << 4);
    // PV: lane (block gb, sub-lane sl) reads keys kb*32 + h*16 + 4*hl + (sl >> 2) (+8*sec),
    // columns 128w + 32c + 16*(gb & 1) + 4*(sl & 3) .. +3 for column block c
    const int gb = ln.lane >> 4, sl = ln.lane & 15;
    const int kk = 4 * ln.hl + (sl >> 2);
    const int cp = 2 * (gb & 1) + ((sl >> 1) & 1);
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int gk = ((sl >> 2) << 2) | (ln.hl + 2 * sec);   // g(key) of key kk + 8*sec
      ln.pv[sec] = ((kk + 8 * sec) * 1024 + 256 * ln.w + 8 * (sl & 1)) | ((cp ^ gk) << 4);
    }
  }

  // Slots of this wave's keys of tile t, one vector load per lane (see
  // TileSlots); keys past the end of the chunk take the last key's slot (a
  // valid index; masked in the math).
  const int ntiles = ntp + ntt;
  auto load_slots = [&](int t) {
    // prefix tiles first, then tree tiles; keys past the end of either list
    // take its last slot; a tile index past the last tile re-reads it
    t = min(t, ntiles - 1);
    const bool tree = t >= ntp;
    const int* list = tree ? a.tree_slot + t0 : a.prefix_slot + p0;
    const int base = (tree ? (t - ntp) * kKeyTile : kbeg + t * kKeyTile) + 16 * ln.w;
    const int last = tree ? min(n_b, kMaxTree) - 1 : kend - 1;
    TileSlots r;
    r.lat = (uint32_t)list[min(base + (ln.lane & 15), last)];
    r.rope[0] = (uint32_t)list[min(base + (ln.lane >> 3), last)];
    r.rope[1] = (uint32_t)list[min(base + 8 + (ln.lane >> 3), last)];
    return r;
  };

  if (ntt > 0) {
    // Ancestor-or-self sets of this tile's rows as bit masks over the tree
    // keys.  A parent that does not precede its child ends a walk, so a
    // malformed array cannot loop; rows past the request's nodes see the root.
    for (int i = threadIdx.x; i < min(n_b, kMaxTree); i += blockDim.x) par_s[i] = a.parent[t0 + i];
    __syncthreads();
    if (threadIdx.x < kRowTile) {
      const int r = tile * kRowTile + (int)threadIdx.x;
      int j = r < rows_b ? min(r / a.num_heads, min(n_b, kMaxTree) - 1) : 0;
      uint64_t m0 = 0, m1 = 0;
      for (int step = 0; step < kMaxTree && j >= 0; ++step) {
        if (j < 64) m0 |= 1ull << j; else m1 |= 1ull << (j - 64);
        const int p = par_s[j];
        j = (p < j) ? p : -1;
      }
      vis_s[threadIdx.x][0] = m0;
      vis_s[threadIdx.x][1] = m1;
    }
    // made visible by the barrier that starts the first tile
  }

  TileSlots sl_next;
  // put tile 0 into `buf` (item start and restarts)
  auto prime = [&](uint8_t* buf) {
    gather_tile(a.pool, load_slots(0), buf, ln.w, ln.lane);
    sl_next = load_slots(1);
  };
  prime(lds0);
  int t = 0;                 // tile held by the buffer processed next
  bool restart = false;      // workgroup-uniform
  bool have_ref = false;     // workgroup-uniform: the reference m is set
  // one tile: `cur` holds tile t while `nxt` receives tile t+1
  auto half_step = [&](uint8_t* cur, uint8_t* nxt) -> bool {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (restart) {
      restart = false;                 // tile_math has cleared o and l
      t = 0;
      prime(cur);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    } else if (t >= ntiles) {
      return false;
    }
    const bool tree = t >= ntp;
    const int nvalid = tree ? kKeyTile : min(kKeyTile, kend - kbeg - t * kKeyTile);
    const uint64_t vis = tree ? vis_s[row_in_tile][t - ntp] : ~0ull;
    restart = tile_math(cur, x, qf, o, st, !have_ref, nvalid, tree, vis, a.scale_log2, ln, a.pool, sl_next, nxt);
    have_ref = true;
    // slots of tile t+2; their latency hides under the wait for tile t+1
    sl_next = load_slots(t + 2);
    ++t;
    return true;
  };
  for (;;) {
    if (!half_step(lds0, lds1)) break;
    if (!half_step(lds1, lds0)) break;
  }

  // Row sums and references of both row blocks: this wave holds l over its
  // key block for this pair's rows; the partner holds the other key block,
  // the other pair the other rows.
  const float lpair = sum_xor32(st.l);
  lds_barrier();                      // everyone is done reading the last P operands
  x.v[ln.w][0][ln.lane] = make_float4(lpair, st.m, 0.f, 0.f);
  lds_barrier();
  const float4 e1 = x.v[ln.w ^ 1][0][ln.lane], e2 = x.v[ln.w ^ 2][0][ln.lane], e3 = x.v[ln.w ^ 3][0][ln.lane];
  const float l_rb[2] = {lpair + e1.x, e2.x + e3.x};
  const size_t pidx = ((size_t)b * a.row_tiles + tile) * a.max_chunks + s;
  float* po = a.part_o + pidx * (kD4 * kRowTile * 4);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int rit = 32 * (ln.pr ^ rb) + ln.l32;
    if (tile * kRowTile + rit >= rows_b) continue;
    const float inv = 1.0f / l_rb[rb];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d4 = (4 * ln.w + c) * 8 + 2 * rq + ln.hl;
        const f32x16& acc = o[4 * rb + c];
        const float4 v = make_float4(acc[4 * rq] * inv, acc[4 * rq + 1] * inv, acc[4 * rq + 2] * inv,
                                     acc[4 * rq + 3] * inv);
        *(float4*)(po + ((size_t)d4 * kRowTile + rit) * 4) = v;
      }
    }
  }
  if (row_ok && ln.hf == 0 && ln.hl == 0) a.part_lse[pidx * kRowTile + row_in_tile] = st.m * kLn2 + logf(l_rb[0]);
}

}  // namespace

hipError_t launch_prefix_splitkv(const PrefixArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(prefix_splitkv_kernel, dim3(a.grid_items), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace vamla
