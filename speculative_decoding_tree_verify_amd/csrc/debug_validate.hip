// Device-side check of a verify call's index data (VAMLA_FLAG_DEBUG_VALIDATE).
//
// The verify kernels trust the index arrays: slot indices, the parent array
// and the cumulative lengths.  The live service these kernels serve runs under
// graph capture with static buffers ("Mapping the Optimization Landscape for
// DDTree Verify Attention", "Input Knowledge Required to Understand This
// Message", item 5), so a caller cannot always copy its index data to the host
// for vamla_validate.  With the debug flag, this kernel runs first on the same
// stream and checks, on the device, what vamla_validate checks on the host:
//
//   array 0, cu_prefix / cu_tree (index b = request):
//       cu_prefix[0] = cu_tree[0] = 0; 0 <= L_b <= max_prefix;
//       1 <= N_b <= max_tree; cu_prefix[B] and cu_tree[B] equal total_prefix
//       and total_tree (at most those with lengths read on the device);
//   array 1, parent (index = global node t): a request's first node has
//       parent -1, its node i has 0 <= parent < i ("Input Knowledge ...",
//       item 1: each draft token sees its ancestors, so parents precede
//       their children);
//   array 2, prefix_slot_idx (index i < cu_prefix[B]): 0 <= slot < pool_slots;
//   array 3, tree_slot_idx (index t < cu_tree[B]): 0 <= slot < pool_slots.
//
// The first violation in (array, index) order is written to the 16-byte record
// {status, array, index, 0}; the record is all zero when everything holds.
// One workgroup does all of it, so the record needs no clearing beforehand and
// the kernel is capture-safe.  The split and merge kernels read the record and
// do no work (the merge writes NaN) when it is set, so a call with bad indices
// never dereferences them.  The arrays past a bad length are not checked.

#include "kernels.h"

namespace vamla {
namespace {

constexpr int kThreads = 1024;
constexpr int kStatusLengths = -8;   // VAMLA_ERR_INVALID_LENGTHS
constexpr int kStatusTree = -6;      // VAMLA_ERR_INVALID_TREE
constexpr int kStatusSlot = -7;      // VAMLA_ERR_INVALID_SLOT

__device__ __forceinline__ uint64_t key_of(int array, int64_t index) {
  return ((uint64_t)array << 40) | (uint64_t)index;
}

// Smallest key of an out-of-range slot among this thread's share of idx[0, n):
// kBatch independent loads in flight per thread, so one workgroup walks a
// long slot list in few memory round trips.
constexpr int kBatch = 16;
__device__ uint64_t check_slots(const int32_t* idx, int64_t n, int64_t pool_slots, int array, int tid) {
  uint64_t mine = ~0ull;
  for (int64_t base = tid; base < n; base += (int64_t)kThreads * kBatch) {
    int32_t v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t i = base + (int64_t)j * kThreads;
      v[j] = i < n ? idx[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t i = base + (int64_t)j * kThreads;
      if (i < n && (v[j] < 0 || (int64_t)v[j] >= pool_slots)) mine = min(mine, key_of(array, i));
    }
  }
  return mine;
}

__global__ __launch_bounds__(kThreads) void debug_validate_kernel(ValidateArgs a) {
  __shared__ unsigned long long first;
  const int tid = threadIdx.x;
  if (tid == 0) first = ~0ull;
  __syncthreads();
  uint64_t mine = ~0ull;
  const int B = a.batch;
  // lengths
  for (int b = tid; b < B; b += kThreads) {
    const int64_t L = (int64_t)a.cu_prefix[b + 1] - a.cu_prefix[b];
    const int64_t N = (int64_t)a.cu_tree[b + 1] - a.cu_tree[b];
    bool bad = L < 0 || L > a.max_prefix || N < 1 || N > a.max_tree;
    if (b == 0) bad |= a.cu_prefix[0] != 0 || a.cu_tree[0] != 0;
    if (b == B - 1) {
      const int64_t tp = a.cu_prefix[B], tt = a.cu_tree[B];
      bad |= a.device_lengths ? (tp > a.total_prefix || tt > a.total_tree)
                              : (tp != a.total_prefix || tt != a.total_tree);
    }
    if (bad) mine = min(mine, key_of(0, b));
  }
  if (mine != ~0ull) atomicMin(&first, (unsigned long long)mine);
  __syncthreads();
  if (first == ~0ull) {
    // the lengths hold, so the arrays below can be indexed with them
    for (int b = tid; b < B; b += kThreads) {
      const int t0 = a.cu_tree[b], n = a.cu_tree[b + 1] - t0;
      for (int i = 0; i < n; ++i) {
        const int p = a.parent[t0 + i];
        if (i == 0 ? p != -1 : (p < 0 || p >= i)) {
          mine = min(mine, key_of(1, t0 + i));
          break;
        }
      }
    }
    mine = min(mine, check_slots(a.prefix_slot, a.cu_prefix[B], a.pool_slots, 2, tid));
    mine = min(mine, check_slots(a.tree_slot, a.cu_tree[B], a.pool_slots, 3, tid));
    if (mine != ~0ull) atomicMin(&first, (unsigned long long)mine);
  }
  __syncthreads();
  if (tid == 0) {
    const uint64_t f = first;
    int4 rec = make_int4(0, 0, 0, 0);
    if (f != ~0ull) {
      const int array = (int)(f >> 40);
      rec.x = array == 0 ? kStatusLengths : array == 1 ? kStatusTree : kStatusSlot;
      rec.y = array;
      rec.z = (int)(f & ((1ull << 40) - 1));
    }
    *(int4*)a.record = rec;
  }
}

}  // namespace

hipError_t launch_debug_validate(const ValidateArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(debug_validate_kernel, dim3(1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace vamla
