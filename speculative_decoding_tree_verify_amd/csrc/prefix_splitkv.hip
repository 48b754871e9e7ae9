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
// prefix key, so the pass is a dense contraction and runs on MFMA.
//
// Waves form two pairs.  Pair p owns query rows [32p, 32p+32) of the tile; the
// two waves of a pair split the work of each 64-key tile:
//   * QK: wave (p, h) computes S^T = K Q^T for keys [32h, 32h+32) of the tile
//     on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS via ds_read_b128, B = the
//     pair's 32 query rows, held in VGPRs for the whole item).  In the 32x32
//     accumulator layout each lane owns one query row.
//   * softmax: P = exp2(S*scale*log2e - m) in bf16, written to LDS so the
//     partner can read it as its own MFMA operand, lane for lane.
//   * PV: wave (p, h) accumulates O^T += V^T P^T for output columns
//     [256h, 256h+256) over all 64 keys (A = V^T read from the same LDS tile by
//     the transposing ds_read_b64_tr_b16, B = own P and the partner's P).
// A wave thus holds 32x576 Q (144 VGPRs) and a 32x256 accumulator (128), which
// leaves the compiler room; LDS bytes per MFMA flop equal those of one wave
// doing all 512 columns.
//
// Gather: the 1152-byte pool row of each key is fetched as 72 sixteen-byte
// pieces with global_load_lds_dwordx4 (straight into LDS, no VGPR staging).
// LDS tile layout is piece-major: byte(key, c) = (c*64 + (key ^ 8*(c&1)))*16,
// which keeps both the ds_read_b128 (QK) and ds_read_b64_tr_b16 (PV) patterns
// free of bank conflicts.  Tiles are double-buffered: the gather of tile t+1
// runs under the math of tile t.
//
// Softmax reference: each row keeps a reference max m.  It only moves when a
// tile's max exceeds it by more than kSlack (log2 units); until then
// exp2(s - m) <= 2^kSlack, well inside bf16/fp32 range, and the O rescale stays
// off the common path.  Moving it is a workgroup-uniform decision, taken after
// the P exchange, with P recomputed from the kept scores.

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
constexpr float kSlack = 16.0f;     // reference max may lag the true max by this much (log2 units)
constexpr float kClamp = 24.0f;     // P exponent cap for the speculative pass

// LDS: two key tiles + exchange area
struct __attribute__((aligned(16))) Xchg {
  // [wave][slot][lane]: slots 0, 1 = the two P operands of the wave's keys;
  // slot 2 = (tile max of the lane's row, move flag, -, -) as four floats
  bf16x8 p[4][3][64];
  float lsum[4][64];                // [wave][lane] final row-sum shares
};

// Workgroup barrier that waits only for this wave's LDS operations.  A fence
// would also wait for the in-flight gathers (LDS DMA counts as LDS stores),
// which must keep running under the math.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8 tr_pair(const uint8_t* base, int off1, int off2) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off1));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off2));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Issue this wave's 18 pieces (c = w, w+4, ..., w+68) of one key tile.
__device__ __forceinline__ void gather_tile(const uint16_t* rowp, uint8_t* lds, int w) {
#pragma unroll
  for (int j = 0; j < kChunks16 / 4; ++j) {
    const int c = w + 4 * j;
    __builtin_amdgcn_global_load_lds((const void*)(rowp + c * 8), (lds_void*)(lds + c * 1024), 16, 0, 0);
  }
}

struct Lane {
  int w, pr, hf, hl, l32, lane;
  int qk_off, trb1, trb2;
};

struct RowState {
  float m;   // reference max of scaled scores (log2 units), shared by the pair
  float l;   // this lane's share of the row sum
};

__device__ __forceinline__ void pack_p(const f32x16& v, float m, bf16x8 (&pb)[2], float& lsum, float cap) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(fminf(v[half * 8 + e] - m, cap));
      lsum += p;
      pb[half][e] = (__bf16)p;
    }
  }
}

// One staged 64-key tile for this wave.
__device__ __forceinline__ void tile_math(const uint8_t* lds, Xchg& x, const bf16x8 (&qf)[36],
                                          f32x16 (&o)[8], RowState& st, int nvalid, float scale_log2,
                                          const Lane& ln) {
  // S^T for this wave's 32 keys
  f32x16 v = {};
#pragma unroll
  for (int s = 0; s < 36; ++s) {
    const bf16x8 a = *(const bf16x8*)(lds + ln.qk_off + s * 2048);
    v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], v, 0, 0, 0);
  }
  // lane holds keys 32*hf + 8*(r/4) + 4*hl + r%4 of row l32
  float mt = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float t = v[r] * scale_log2;
    if (32 * ln.hf + 8 * (r >> 2) + 4 * ln.hl + (r & 3) >= nvalid) t = -INFINITY;
    v[r] = t;
    mt = fmaxf(mt, t);
  }
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  // speculative P against the current reference
  float lsum = 0.f;
  bf16x8 pb[2];
  pack_p(v, st.m, pb, lsum, kClamp);
  x.p[ln.w][0][ln.lane] = pb[0];
  x.p[ln.w][1][ln.lane] = pb[1];
  const float want = __any(mt > st.m + kSlack) ? 1.f : 0.f;
  x.p[ln.w][2][ln.lane] = __builtin_bit_cast(bf16x8, make_float4(mt, want, 0.f, 0.f));
  lds_barrier();
  auto aux = [&](int w, int l) { return __builtin_bit_cast(float4, x.p[w][2][l]); };
  // each writer stored its wave-uniform flag in every lane, so read at own lane
  const float any_flag = aux(0, ln.lane).y + aux(1, ln.lane).y + aux(2, ln.lane).y + aux(3, ln.lane).y;
  if (__builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, any_flag)) != 0) {
    // move the pair's reference to the pair's tile max (rare: first tile, or a
    // jump of more than kSlack); both waves of the pair compute the same m_new
    const float m_new = fmaxf(st.m, fmaxf(mt, aux(ln.w ^ 1, ln.lane).x));
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] *= alpha;
    lsum = 0.f;
    pack_p(v, st.m, pb, lsum, INFINITY);
    lds_barrier();
    x.p[ln.w][0][ln.lane] = pb[0];
    x.p[ln.w][1][ln.lane] = pb[1];
    lds_barrier();
  }
  st.l += lsum;
  const bf16x8 pq0 = x.p[ln.w ^ 1][0][ln.lane];
  const bf16x8 pq1 = x.p[ln.w ^ 1][1][ln.lane];
  // O^T += V^T P^T for this wave's 256 output columns over all 64 keys
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int dblk = 8 * ln.hf + j;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int off = dblk * 4096 + kb * 512 + half * 256;
        const bf16x8 a = tr_pair(lds, ln.trb1 + off, ln.trb2 + off);
        const bf16x8 bop = (kb == ln.hf) ? pb[half] : (half ? pq1 : pq0);
        o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, o[j], 0, 0, 0);
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void prefix_splitkv_kernel(PrefixArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kTileBytes];
  __shared__ Xchg x;
  // [tile & 1][key]: slot indices of an upcoming tile.  Its own LDS object, so
  // the compiler can tell the DMA into it from the exchange area's traffic.
  __shared__ uint32_t slot_ring[2][64];

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
  const int kbeg = s * a.chunk;
  if (kbeg >= L) return;
  const int kend = min(kbeg + a.chunk, L);
  const int t0 = a.cu_tree[b];
  const int rows_b = (a.cu_tree[b + 1] - t0) * a.num_heads;
  if (tile * kRowTile >= rows_b) return;

  const int row_in_tile = ln.pr * 32 + ln.l32;
  const int row = tile * kRowTile + row_in_tile;
  const bool row_ok = row < rows_b;

  // the pair's query rows: lane (l32, hl) holds pieces 2s+hl of row l32
  bf16x8 qf[36];
  {
    const uint16_t* qrow = a.q + ((size_t)t0 * a.num_heads + (row_ok ? row : 0)) * kDqk;
#pragma unroll
    for (int s2 = 0; s2 < 36; ++s2) {
      bf16x8 v = *(const bf16x8*)(qrow + (2 * s2 + ln.hl) * 8);
      qf[s2] = row_ok ? v : bf16x8{};
    }
  }

  f32x16 o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x16{};
  RowState st{-INFINITY, 0.f};

  // lane constants for LDS reads
  ln.qk_off = ln.hf * 512 + ln.hl * 1024 + ((ln.l32 ^ (8 * ln.hl)) * 16);
  {
    const int g = ln.lane >> 4, sl = ln.lane & 15;
    const int cpart = 2 * (g & 1) + ((sl >> 1) & 1);
    const int xr = 8 * ((sl >> 1) & 1);
    const int keyoff = 4 * ln.hl + (sl >> 2);
    ln.trb1 = cpart * 1024 + 8 * (sl & 1) + (keyoff + xr) * 16;
    ln.trb2 = cpart * 1024 + 8 * (sl & 1) + (keyoff + (8 - xr)) * 16;
  }

  // gather lane: this wave writes pieces of parity (w & 1), so lane loads key lane ^ 8*(w&1)
  const int gkey = ln.lane ^ (8 * (ln.w & 1));
  const int* slots = a.prefix_slot + p0;
  const int ntiles = (kend - kbeg + kKeyTile - 1) / kKeyTile;
  auto row_of = [&](uint32_t slot) -> const uint16_t* { return a.pool + (size_t)slot * kDqk; };
  // Slot indices travel to LDS by DMA too, two tiles ahead of their use, so no
  // register waits on them while gathers are in flight.  Keys past the end of
  // the chunk read the last key's slot (a valid index; masked in the math).
  auto slot_dma = [&](int t) {
    const int key = min(kbeg + t * kKeyTile + ln.lane, kend - 1);
    __builtin_amdgcn_global_load_lds((const void*)(slots + key), (lds_void*)&slot_ring[t & 1][0], 4, 0, 0);
  };

  gather_tile(row_of((uint32_t)slots[min(kbeg + gkey, kend - 1)]), lds0, ln.w);
  if (ln.w == 0) slot_dma(1);

  for (int t = 0; t < ntiles; t += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles) {
      gather_tile(row_of(slot_ring[1][gkey]), lds1, ln.w);
      if (ln.w == 0) slot_dma(t + 2);
    }
    tile_math(lds0, x, qf, o, st, min(kKeyTile, kend - kbeg - t * kKeyTile), a.scale_log2, ln);
    if (t + 1 >= ntiles) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < ntiles) {
      gather_tile(row_of(slot_ring[0][gkey]), lds0, ln.w);
      if (ln.w == 0) slot_dma(t + 3);
    }
    tile_math(lds1, x, qf, o, st, min(kKeyTile, kend - kbeg - (t + 1) * kKeyTile), a.scale_log2, ln);
  }

  // row sum: own lane, lane ^ 32, and the partner's two lanes
  const float lpair = st.l + __shfl_xor(st.l, 32);
  x.lsum[ln.w][ln.lane] = lpair;
  lds_barrier();
  const float l_tot = lpair + x.lsum[ln.w ^ 1][ln.lane];
  if (!row_ok) return;
  const float inv = 1.0f / l_tot;
  const size_t pidx = ((size_t)b * a.row_tiles + tile) * a.max_chunks + s;
  float* po = a.part_o + pidx * (kD4 * kRowTile * 4);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int dblk = 8 * ln.hf + j;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d4 = dblk * 8 + 2 * rq + ln.hl;
      float4 v = make_float4(o[j][4 * rq] * inv, o[j][4 * rq + 1] * inv, o[j][4 * rq + 2] * inv,
                             o[j][4 * rq + 3] * inv);
      *(float4*)(po + ((size_t)d4 * kRowTile + row_in_tile) * 4) = v;
    }
  }
  if (ln.hf == 0 && ln.hl == 0) a.part_lse[pidx * kRowTile + row_in_tile] = st.m * kLn2 + logf(l_tot);
}

}  // namespace

hipError_t launch_prefix_splitkv(const PrefixArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(prefix_splitkv_kernel, dim3(a.grid_items), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace vamla
