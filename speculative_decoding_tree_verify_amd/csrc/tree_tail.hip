// Masked tree-tail attention for DDTree verify (gfx950).
//
// Each tree node attends, besides the prefix, to itself and its ancestors in
// the drafted tree ("Mapping the Optimization Landscape for DDTree Verify
// Attention", "Input Knowledge Required to Understand This Message", item 1;
// read as ancestors-or-self).  This pass computes, for every node and head, the
// normalised partial (o_tail, lse_tail) over that visible tree set only; the
// merge pass combines it with the prefix partials ("The Architecture Detective:
// Uncovering FlashMLA's Potential for Blackwell DDTree Verification", "The
// Message in Full": a small custom kernel for the masked tree tail, tiny since
// q_len <= 65).
//
// One 256-thread workgroup per node: walk the parent array to the root, stage
// the <= 65 visible latent rows in LDS, then all H heads' scores, softmax and
// P.V in fp32.  The work is a few MFLOP per step, so plain FMA is enough.

#include "kernels.h"

namespace vamla {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ __launch_bounds__(256) void tree_tail_kernel(TailArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t krow[kMaxTree][kDqk];   // visible rows
  __shared__ float w[kMaxHeads][kMaxTree + 1];                           // scores -> weights
  __shared__ float lse_h[kMaxHeads];
  __shared__ int anc[kMaxTree];
  __shared__ int n_anc;

  const int tg = blockIdx.x;          // global node index
  const int H = a.num_heads;
  // request owning node tg: last b with cu_tree[b] <= tg
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_tree[mid] <= tg) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int t0 = a.cu_tree[b];
  const int tl = tg - t0;

  if (threadIdx.x == 0) {
    // ancestors-or-self; a parent that does not precede its child ends the walk,
    // so a malformed array cannot loop
    int n = 0, j = tl;
    while (j >= 0 && n < kMaxTree) {
      anc[n++] = j;
      const int p = a.parent[t0 + j];
      j = (p < j) ? p : -1;
    }
    n_anc = n;
  }
  __syncthreads();
  const int na = n_anc;

  for (int i = threadIdx.x; i < na * kChunks16; i += blockDim.x) {
    const int r = i / kChunks16, c = i - r * kChunks16;
    const uint32_t slot = (uint32_t)a.tree_slot[t0 + anc[r]];
    *(uint4*)&krow[r][c * 8] = *(const uint4*)(a.pool + (size_t)slot * kDqk + c * 8);
  }
  __syncthreads();

  // scores s[h][r] = scale * <q[tg,h,:], K[anc r]>
  for (int i = threadIdx.x; i < H * na; i += blockDim.x) {
    const int h = i / na, r = i - h * na;
    const uint4* qv = (const uint4*)(a.q + ((size_t)tg * H + h) * kDqk);
    const uint4* kv = (const uint4*)&krow[r][0];
    float acc = 0.f;
#pragma unroll 4
    for (int c = 0; c < kChunks16; ++c) {
      const uint4 x = qv[c], y = kv[c];
      acc = fmaf(bf16_lo(x.x), bf16_lo(y.x), acc);
      acc = fmaf(bf16_hi(x.x), bf16_hi(y.x), acc);
      acc = fmaf(bf16_lo(x.y), bf16_lo(y.y), acc);
      acc = fmaf(bf16_hi(x.y), bf16_hi(y.y), acc);
      acc = fmaf(bf16_lo(x.z), bf16_lo(y.z), acc);
      acc = fmaf(bf16_hi(x.z), bf16_hi(y.z), acc);
      acc = fmaf(bf16_lo(x.w), bf16_lo(y.w), acc);
      acc = fmaf(bf16_hi(x.w), bf16_hi(y.w), acc);
    }
    w[h][r] = acc * a.scale;
  }
  __syncthreads();

  // softmax over the visible set, per head
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    float m = -INFINITY;
    for (int r = 0; r < na; ++r) m = fmaxf(m, w[h][r]);
    float sum = 0.f;
    for (int r = 0; r < na; ++r) {
      const float e = __expf(w[h][r] - m);
      w[h][r] = e;
      sum += e;
    }
    const float inv = 1.f / sum;
    for (int r = 0; r < na; ++r) w[h][r] *= inv;
    lse_h[h] = m + logf(sum);
  }
  __syncthreads();

  // o[h][4 d4 .. 4 d4 + 3] = sum_r w[h][r] * V[r][...]; written in the merge layout
  for (int i = threadIdx.x; i < H * kD4; i += blockDim.x) {
    const int h = i / kD4, d4 = i - h * kD4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = 0; r < na; ++r) {
      const uint2 v = *(const uint2*)&krow[r][d4 * 4];
      const float wr = w[h][r];
      acc.x = fmaf(wr, bf16_lo(v.x), acc.x);
      acc.y = fmaf(wr, bf16_hi(v.x), acc.y);
      acc.z = fmaf(wr, bf16_lo(v.y), acc.z);
      acc.w = fmaf(wr, bf16_hi(v.y), acc.w);
    }
    const int rr = tl * H + h;                 // row within the request
    const int tile = rr / kRowTile, rit = rr - tile * kRowTile;
    if (tile >= a.row_tiles) continue;         // more nodes than max_tree: caller error, stay in bounds
    const size_t base = (size_t)b * a.row_tiles + tile;
    *(float4*)(a.tail_o + ((base * kD4 + d4) * kRowTile + rit) * 4) = acc;
    if (d4 == 0) a.tail_lse[base * kRowTile + rit] = lse_h[h];
  }
}

}  // namespace

hipError_t launch_tree_tail(const TailArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(tree_tail_kernel, dim3(a.total_tree), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace vamla
