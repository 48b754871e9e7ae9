// Scattered-row read rate: the pool rows a split pass gathers, read with
// nothing else done to them.
//
// The pages measure a verify kernel by its effective KV-read bandwidth
// against the HBM peak ("The Anatomy of a Kernel Investigation", "Phase 3";
// "The Architecture Detective ...", "Performance Analysis").  Rows of a
// page_size=1 pool are 1152-byte runs at random slots, which no kernel reads
// at the rate of a contiguous stream; this kernel measures the rate a plain
// read of exactly those rows reaches, the practical ceiling for the split
// pass in its HBM-bound regime.  Each thread reads 16-byte pieces of rows
// (72 per row, 8 rows per 576-thread block, kUnroll rows of the block's
// stride in flight per thread) and folds them into one 32-bit XOR; each wave
// XOR-reduces its lanes and writes one sink word, so the XOR of all sink words
// equals the XOR of every 32-bit word of the n rows (a check that every row
// was read).  64-bit row offsets (pools beyond 4 GiB).

#include "kernels.h"
#include "vamla.h"

namespace vamla {
namespace {

constexpr int kRowsPerBlock = 8;
constexpr int kThreads = kRowsPerBlock * kChunks16;   // 576: nine waves
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void read_rows_kernel(const uint4* __restrict__ pool,
                                                             const int32_t* __restrict__ idx, int64_t n,
                                                             uint32_t* __restrict__ sink) {
  const int rl = threadIdx.x / kChunks16;
  const int c = threadIdx.x - rl * kChunks16;
  const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
  uint32_t acc = 0;
  for (int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock + rl; r0 < n; r0 += stride * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t r = r0 + u * stride;
      v[u] = r < n ? pool[(uint64_t)(uint32_t)idx[r] * kChunks16 + c] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= (v[u].x ^ v[u].y) ^ (v[u].z ^ v[u].w);
  }
  for (int m = 1; m < 64; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_read_rows(const uint16_t* pool, const int32_t* idx, int64_t n, uint32_t* sink,
                            hipStream_t stream) {
  static_assert(kReadRowsBlocks * (kThreads / 64) == VAMLA_READ_ROWS_SINK_WORDS, "sink size");
  hipLaunchKernelGGL(read_rows_kernel, dim3(kReadRowsBlocks), dim3(kThreads), 0, stream, (const uint4*)pool, idx,
                     n, sink);
  return hipGetLastError();
}

}  // namespace vamla
