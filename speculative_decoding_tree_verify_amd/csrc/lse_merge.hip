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
// Layout: partials are [item][128 d4][64 rows][4 floats], so thread = row reads
// coalesced 16-byte pieces; grid = (request x row tile) x column groups.

#include "kernels.h"

namespace vamla {
namespace {

constexpr int kD4PerBlock = 4;   // float4 column groups per thread

__global__ __launch_bounds__(kRowTile) void lse_merge_kernel(MergeArgs a) {
  const int item = blockIdx.x;
  const int b = item / a.row_tiles;
  const int tile = item - b * a.row_tiles;
  const int t0 = a.cu_tree[b];
  const int rows_b = (a.cu_tree[b + 1] - t0) * a.num_heads;
  const int rit = threadIdx.x;
  const int r = tile * kRowTile + rit;
  if (r >= rows_b) return;
  const int L = a.cu_prefix[b + 1] - a.cu_prefix[b];
  // a prefix longer than max_prefix is a caller error; never read past the plan
  const int S = max(1, min((L + a.chunk - 1) / a.chunk, a.max_chunks));

  const size_t tb = (size_t)b * a.row_tiles + tile;
  const size_t p0 = tb * a.max_chunks;
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, a.part_lse[(p0 + s) * kRowTile + rit]);
  float sum = 0.f;
  for (int s = 0; s < S; ++s) sum += __expf(a.part_lse[(p0 + s) * kRowTile + rit] - m);
  const float lse = m + logf(sum);

  const size_t orow = (size_t)t0 * a.num_heads + r;   // global row (t, h)
  if (blockIdx.y == 0) a.lse[orow] = lse;

  const int d4_0 = blockIdx.y * kD4PerBlock;
  float4 acc[kD4PerBlock];
#pragma unroll
  for (int j = 0; j < kD4PerBlock; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; ++s) {
    const float ws = __expf(a.part_lse[(p0 + s) * kRowTile + rit] - lse);
#pragma unroll
    for (int j = 0; j < kD4PerBlock; ++j) {
      const float4 v = *(const float4*)(a.part_o + (((p0 + s) * kD4 + d4_0 + j) * kRowTile + rit) * 4);
      acc[j].x = fmaf(ws, v.x, acc[j].x);
      acc[j].y = fmaf(ws, v.y, acc[j].y);
      acc[j].z = fmaf(ws, v.z, acc[j].z);
      acc[j].w = fmaf(ws, v.w, acc[j].w);
    }
  }
  // bf16, round to nearest even
  uint16_t* o = a.out + orow * kDv + d4_0 * 4;
#pragma unroll
  for (int j = 0; j < kD4PerBlock; ++j) {
    const __bf16 h0 = (__bf16)acc[j].x, h1 = (__bf16)acc[j].y, h2 = (__bf16)acc[j].z, h3 = (__bf16)acc[j].w;
    uint2 pk;
    pk.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    pk.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
    *(uint2*)(o + j * 4) = pk;
  }
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(lse_merge_kernel, dim3(a.batch * a.row_tiles, kD4 / kD4PerBlock), dim3(kRowTile), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace vamla
