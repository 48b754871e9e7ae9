// Slot compaction (defragmentation) gather: dst[l, :] = pool[idx[l], :].
//
// A page_size=1 pool scatters a request's rows once the free list has churned
// ("The Architecture Detective: Uncovering FlashMLA's Potential for Blackwell
// DDTree Verification", "Defragmentation: Separating Signal from Noise").
// Copying the rows of a request into a contiguous run lets the verify pass be
// compared on scrambled and contiguous pools.  Pure byte movement: each thread
// copies one 16-byte piece, 72 pieces per 1152-byte row, with 64-bit offsets
// (pools beyond 4 GiB).  HBM-bound: 2 x 1152 bytes per row.

#include "kernels.h"

namespace vamla {
namespace {

constexpr int kRowsPerBlock = 8;

__global__ __launch_bounds__(kRowsPerBlock * kChunks16) void slot_gather_kernel(const uint4* __restrict__ pool,
                                                                                 const int32_t* __restrict__ idx,
                                                                                 int64_t n, uint4* __restrict__ dst) {
  const int rl = threadIdx.x / kChunks16;
  const int c = threadIdx.x - rl * kChunks16;
  for (int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock; r0 < n; r0 += (int64_t)gridDim.x * kRowsPerBlock) {
    const int64_t r = r0 + rl;
    if (r < n) {
      const uint64_t src = (uint64_t)(uint32_t)idx[r] * kChunks16 + c;
      dst[r * kChunks16 + c] = pool[src];
    }
  }
}

}  // namespace

hipError_t launch_slot_gather(const uint16_t* pool, const int32_t* idx, int64_t n, uint16_t* dst,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(slot_gather_kernel, dim3((unsigned)blocks), dim3(kRowsPerBlock * kChunks16), 0, stream,
                     (const uint4*)pool, idx, n, (uint4*)dst);
  return hipGetLastError();
}

}  // namespace vamla
