// Log-sum-exp merge of split attention partials (gfx950).
//
// The split pass leaves one normalised partial (o_s, lse_s) per prefix chunk
// of a request, the last one covering the request's tree keys as well (a
// request with no prefix has one partial, over its tree).  The exact attention
// over their union is
//     lse = ln( sum_s exp(lse_s) ),   out = sum_s exp(lse_s - lse) * o_s,
// the merge of partial attention states the split design relies on ("The
// Anatomy of a Kernel Investigation", "The Reasoning Process: A Deep Dive",
// Phase 2; "The Architecture Detective: ...", "The Message in Full").
// Chunks past a request's prefix were never written and are not read.
//
// Layout: partials are [item][128 d4][64 rows][4 floats], so for one chunk
// and one float4 column group the rows of a tile are 1 KB of contiguous
// memory.  A 256-thread workgroup covers one row tile and 4 / CW column
// groups, CW waves per column group (CW = 1, 2 or 4).  A wave's 64 lanes are
// RL rows x CL chunk lanes (RL = the tile's live rows rounded up to a power
// of two, at most 64; RL * CL = 64), so every load instruction reads CL
// segments of RL * 16 >= 64 contiguous bytes.  Thread (chunk wave cw, chunk
// lane c) takes chunks k, k + CW*CL, ... with k = cw * CL + c, folds them with
// a running max (the loads of a batch in flight together), and the partial
// states (max, sum, float4) are combined across chunk lanes by lane shuffles
// and across the CW waves through LDS.  With few rows and many chunks
// (decode-like calls) this keeps 128 workgroups per row tile busy instead of
// a handful of lanes walking every chunk in turn; with many row tiles the
// host takes CW = 1 and RL = 64, one wave per column group and no exchange.

#include "kernels.h"

namespace vamla {
namespace {

constexpr int kWaves = 4;
constexpr int kBatch = 16;          // chunks whose loads a thread issues together

struct State {
  float m, s;
  float4 a;
};

__device__ __forceinline__ void fold(State& x, const State& y) {
  const float M = fmaxf(x.m, y.m);
  // an empty state (m = -inf) has weight 0; two empty states stay empty
  const float cx = x.m == -INFINITY ? 0.f : __expf(x.m - M);
  const float cy = y.m == -INFINITY ? 0.f : __expf(y.m - M);
  x.s = x.s * cx + y.s * cy;
  x.a.x = x.a.x * cx + y.a.x * cy;
  x.a.y = x.a.y * cx + y.a.y * cy;
  x.a.z = x.a.z * cx + y.a.z * cy;
  x.a.w = x.a.w * cx + y.a.w * cy;
  x.m = M;
}

__device__ __forceinline__ State shfl_state(const State& x, int mask) {
  State y;
  y.m = __shfl_xor(x.m, mask);
  y.s = __shfl_xor(x.s, mask);
  y.a.x = __shfl_xor(x.a.x, mask);
  y.a.y = __shfl_xor(x.a.y, mask);
  y.a.z = __shfl_xor(x.a.z, mask);
  y.a.w = __shfl_xor(x.a.w, mask);
  return y;
}

__global__ __launch_bounds__(64 * kWaves) void lse_merge_kernel(MergeArgs a) {
  __shared__ State red[kWaves][kRowTile];
  // every kernel-argument load issued at once (see the split kernel: the
  // compiler would otherwise load these only after the debug test's load)
  asm volatile("" ::"s"(a.part_o), "s"(a.part_lse), "s"(a.cu_prefix), "s"(a.cu_tree), "s"(a.chunk_wave_bits),
               "s"(a.device_lengths));
  if (a.debug_record && __builtin_amdgcn_readfirstlane(a.debug_record[0]) != 0) {
    // the index data failed the device-side check: every output is NaN (the
    // lengths may be what failed, so rows are covered by the call's totals)
    const int64_t rows = (int64_t)a.total_tree * a.num_heads;
    const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    const int64_t gid = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    const uint2 nan2 = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
    for (int64_t i = gid; i < rows * (kDv / 4); i += nthreads) *(uint2*)(a.out + i * 4) = nan2;
    for (int64_t i = gid; i < rows; i += nthreads) a.lse[i] = __builtin_nanf("");
    return;
  }
  const int item = blockIdx.x;
  const int b = item / a.row_tiles;
  const int tile = item - b * a.row_tiles;
  const int cw_bits = a.chunk_wave_bits;
  const int CW = 1 << cw_bits;
  // a single request's bounds are the call's totals (no load before the
  // partials'), unless the lengths are to be read on the device
  const bool one = a.batch == 1 && !a.device_lengths;
  const int chunk = a.device_lengths ? device_chunk(a.cu_prefix, a.batch, a.max_chunks) : a.chunk;
  const int t0 = one ? 0 : a.cu_tree[b];
  const int rows_b = ((one ? a.total_tree : a.cu_tree[b + 1]) - t0) * a.num_heads;
  if (tile * kRowTile >= rows_b) return;
  const int L = one ? a.total_prefix : a.cu_prefix[b + 1] - a.cu_prefix[b];
  // a prefix longer than max_prefix is a caller error; never read past the plan
  const int S = max(1, min((L + chunk - 1) / chunk, a.max_chunks));

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rl_bits = a.row_bits;
  const int RL = 1 << rl_bits;
  const int CL = 64 >> rl_bits;
  const int rit = lane & (RL - 1);                // row within the tile
  const int cl = lane >> rl_bits;                 // chunk lane
  const int cw = w & (CW - 1);                    // chunk wave
  const int d4 = blockIdx.y * (kWaves >> cw_bits) + (w >> cw_bits);
  const int k0 = cw * CL + cl;
  const int kstep = CW * CL;
  const bool live = tile * kRowTile + rit < rows_b;

  const size_t p0 = ((size_t)b * a.row_tiles + tile) * a.max_chunks;
  const float* lse_p = a.part_lse + p0 * kRowTile + rit;
  const float4* o_p = (const float4*)a.part_o + (p0 * kD4 + d4) * kRowTile + rit;
  const size_t o_stride = (size_t)kD4 * kRowTile;          // float4s per chunk partial

  State st{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
  if (live) {
    for (int s0 = k0; s0 < S; s0 += kBatch * kstep) {
      float4 v[kBatch];
      float lw[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int s = s0 + j * kstep;
        if (s < S) {
          v[j] = o_p[(size_t)s * o_stride];
          lw[j] = lse_p[s * kRowTile];
        }
      }
      float mb = st.m;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (s0 + j * kstep < S) mb = fmaxf(mb, lw[j]);
      if (mb > st.m) {                 // rescale what earlier batches summed
        const float c = __expf(st.m - mb);
        st.s *= c;
        st.a.x *= c;
        st.a.y *= c;
        st.a.z *= c;
        st.a.w *= c;
        st.m = mb;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (s0 + j * kstep < S) {
          const float e = __expf(lw[j] - st.m);
          st.s += e;
          st.a.x = fmaf(e, v[j].x, st.a.x);
          st.a.y = fmaf(e, v[j].y, st.a.y);
          st.a.z = fmaf(e, v[j].z, st.a.z);
          st.a.w = fmaf(e, v[j].w, st.a.w);
        }
      }
    }
  }
  // chunk lanes of a row: lanes rit + RL * c, c = 0 .. CL-1
  for (int mask = RL; mask < 64; mask <<= 1) fold(st, shfl_state(st, mask));
  if (CW > 1) {
    if (cl == 0) red[w][rit] = st;
    __syncthreads();
    for (int i = 1; i < CW; ++i)
      if (cw == 0) fold(st, red[w + i][rit]);
  }
  if (cw != 0 || cl != 0 || !live) return;

  const float inv = 1.f / st.s;
  const size_t orow = (size_t)t0 * a.num_heads + tile * kRowTile + rit;   // global row (t, h)
  if (d4 == 0) a.lse[orow] = st.m + logf(st.s);
  // bf16, round to nearest even
  const __bf16 h0 = (__bf16)(st.a.x * inv), h1 = (__bf16)(st.a.y * inv), h2 = (__bf16)(st.a.z * inv),
               h3 = (__bf16)(st.a.w * inv);
  uint2 pk;
  pk.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  pk.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
  *(uint2*)(a.out + orow * kDv + d4 * 4) = pk;
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.row_bits < 0 || a.row_bits > 6 || a.chunk_wave_bits < 0 || a.chunk_wave_bits > 2) return hipErrorInvalidValue;
  const dim3 grid(a.batch * a.row_tiles, (kD4 / kWaves) << a.chunk_wave_bits), block(64 * kWaves);
  hipLaunchKernelGGL(lse_merge_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace vamla
