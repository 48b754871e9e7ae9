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
// Layout: partials are [item][128 d4][64 rows][4 floats].  A 256-thread
// workgroup covers one row tile and four float4 column groups; thread =
// (column group, row), so each wave reads one coalesced 1 KB piece per chunk.
// Every thread keeps its chunks' loads in flight at once: the pass is a
// stream over the partials and needs many waves per CU to reach HBM speed.

#include "kernels.h"

namespace vamla {
namespace {

constexpr int kGroups = 4;          // float4 column groups per workgroup

// kBatch = chunks whose loads are issued together (16 or 32; fewer registers
// when the plan has at most 16 chunks)
template <int kBatch>
__global__ __launch_bounds__(kRowTile * kGroups) void lse_merge_kernel(MergeArgs a) {
  const int item = blockIdx.x;
  const int b = item / a.row_tiles;
  const int tile = item - b * a.row_tiles;
  // a single request's bounds are the call's totals (no load before the partials')
  const bool one = a.batch == 1;
  const int t0 = one ? 0 : a.cu_tree[b];
  const int rows_b = ((one ? a.total_tree : a.cu_tree[b + 1]) - t0) * a.num_heads;
  const int rit = threadIdx.x & (kRowTile - 1);
  const int d4 = blockIdx.y * kGroups + (threadIdx.x >> 6);
  const int r = tile * kRowTile + rit;
  if (r >= rows_b) return;
  const int L = one ? a.total_prefix : a.cu_prefix[b + 1] - a.cu_prefix[b];
  // a prefix longer than max_prefix is a caller error; never read past the plan
  const int S = max(1, min((L + a.chunk - 1) / a.chunk, a.max_chunks));

  const size_t p0 = ((size_t)b * a.row_tiles + tile) * a.max_chunks;
  const float* lse_p = a.part_lse + p0 * kRowTile + rit;
  const float4* o_p = (const float4*)a.part_o + (p0 * kD4 + d4) * kRowTile + rit;
  const size_t o_stride = (size_t)kD4 * kRowTile;          // float4s per chunk partial

  // One round trip: the chunks' lse values and partials are loaded
  // together, the max is taken from registers.  Requests with more chunks
  // than fit in one batch fold their batches with a running max.
  float m = -INFINITY;
  float sum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float4 v[kBatch];
    float w[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < S) {
        v[j] = o_p[(size_t)(s0 + j) * o_stride];
        w[j] = lse_p[(s0 + j) * kRowTile];
      }
    }
    float mb = m;
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < S) mb = fmaxf(mb, w[j]);
    if (mb > m) {                    // rescale what earlier batches summed
      const float c = __expf(m - mb);
      sum *= c;
      acc.x *= c;
      acc.y *= c;
      acc.z *= c;
      acc.w *= c;
      m = mb;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < S) {
        const float e = __expf(w[j] - m);
        sum += e;
        acc.x = fmaf(e, v[j].x, acc.x);
        acc.y = fmaf(e, v[j].y, acc.y);
        acc.z = fmaf(e, v[j].z, acc.z);
        acc.w = fmaf(e, v[j].w, acc.w);
      }
    }
  }
  const float inv = 1.f / sum;
  const size_t orow = (size_t)t0 * a.num_heads + r;   // global row (t, h)
  if (d4 == 0) a.lse[orow] = m + logf(sum);
  // bf16, round to nearest even
  const __bf16 h0 = (__bf16)(acc.x * inv), h1 = (__bf16)(acc.y * inv), h2 = (__bf16)(acc.z * inv),
               h3 = (__bf16)(acc.w * inv);
  uint2 pk;
  pk.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  pk.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
  *(uint2*)(a.out + orow * kDv + d4 * 4) = pk;
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
  const dim3 grid(a.batch * a.row_tiles, kD4 / kGroups), block(kRowTile * kGroups);
  if (a.max_chunks <= 16)
    hipLaunchKernelGGL(lse_merge_kernel<16>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(lse_merge_kernel<32>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace vamla
