// Internal declarations shared by the HIP kernels and the host library.
// Not part of the public ABI (include/vamla.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vamla {

constexpr int kDqk = 576;                  // latent 512 + rope 64
constexpr int kDv = 512;
constexpr int kChunks16 = kDqk / 8;        // 72 sixteen-byte pieces per pool row
constexpr int kKeyTile = 32;               // chunk sizes are multiples of this (the key tile)
constexpr int kRowTile = 64;               // query rows per split work item
constexpr int kD4 = kDv / 4;               // 128 float4 groups per output row
constexpr int kMaxTree = 65;
constexpr int kMaxHeads = 128;

// Split-KV pass: prefix chunks, the last one of each request with its tree keys.
struct PrefixArgs {
  const uint16_t* q;          // [T, H, 576] bf16
  const uint16_t* pool;       // [P, 576] bf16
  const int32_t* prefix_slot; // [total_prefix]
  const int32_t* tree_slot;   // [T]
  const int32_t* parent;      // [T], request-local
  const int32_t* cu_prefix;   // [B+1]
  const int32_t* cu_tree;     // [B+1]
  float* part_o;              // [B][row_tiles][max_chunks][128 d4][64 rows][4]
  float* part_lse;            // [B][row_tiles][max_chunks][64 rows]
  int32_t num_heads;
  int32_t chunk;
  int32_t row_tiles;
  int32_t max_chunks;
  int32_t batch;
  int32_t grid_items;         // multiple of 8
  int32_t total_prefix;       // = cu_prefix[B]; with B = 1 the kernel takes
  int32_t total_tree;         // the request's bounds from these two, not cu_*
  float scale_log2;           // softmax_scale * log2(e)
  int32_t device_lengths;     // 1: lengths from cu_* only, chunk from device_chunk()
  const int32_t* debug_record; // non-null with VAMLA_FLAG_DEBUG_VALIDATE: no work if record[0] != 0
  uint16_t* out;              // non-null when every request is one chunk: the final out [T, H, 512]
  float* lse;                 // and lse [T, H] are written here instead of partials (no merge)
};

// LSE merge of the chunk partials.
struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* cu_prefix;
  const int32_t* cu_tree;
  uint16_t* out;              // [T, H, 512] bf16
  float* lse;                 // [T, H]
  int32_t num_heads;
  int32_t chunk;
  int32_t row_tiles;
  int32_t max_chunks;
  int32_t batch;
  int32_t total_prefix;       // as in PrefixArgs
  int32_t total_tree;
  int32_t row_bits;           // log2 of the rows a wave covers (<= 6): live rows of a tile, rounded up
  int32_t chunk_wave_bits;    // log2 of the waves that split one column group's chunks (<= 2)
  int32_t device_lengths;     // as in PrefixArgs
  const int32_t* debug_record; // as in PrefixArgs; a set record makes the merge write NaN
};

// Device-side check of the index arrays (VAMLA_FLAG_DEBUG_VALIDATE).
struct ValidateArgs {
  const int32_t* cu_prefix;
  const int32_t* cu_tree;
  const int32_t* parent;
  const int32_t* prefix_slot;
  const int32_t* tree_slot;
  int32_t* record;            // int32[4]: status, array, index, 0 (all zero: valid)
  int64_t max_prefix;
  int64_t total_prefix;
  int64_t pool_slots;
  int32_t batch;
  int32_t max_tree;
  int32_t total_tree;
  int32_t device_lengths;
};

// Chunk size chosen on the device from the longest prefix in cu_prefix: the
// smallest multiple of the key tile that splits it into at most max_chunks
// chunks (at least one tile).  Split and merge compute the same value.  Each
// lane reads every 64th request's length (one round of loads in flight
// however large the batch), then the wave takes the max across lanes; every
// lane of the wave must be active.
__device__ __forceinline__ int device_chunk(const int32_t* cu_prefix, int batch, int max_chunks) {
  const int lane = threadIdx.x & 63;
  int lmax = 0;
  for (int i = lane; i < batch; i += 64) lmax = max(lmax, cu_prefix[i + 1] - cu_prefix[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lmax = max(lmax, __shfl_xor(lmax, off));
  const int c = (lmax + max_chunks - 1) / max_chunks;
  return max(kKeyTile, (c + kKeyTile - 1) / kKeyTile * kKeyTile);
}

hipError_t launch_prefix_splitkv(const PrefixArgs& a, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_debug_validate(const ValidateArgs& a, hipStream_t stream);
// Read of n pool rows by slot index, folded into VAMLA_READ_ROWS_SINK_WORDS
// XOR words (a fixed grid of kReadRowsBlocks blocks, two per CU).
constexpr int kReadRowsBlocks = 512;
hipError_t launch_read_rows(const uint16_t* pool, const int32_t* idx, int64_t n, uint32_t* sink,
                            hipStream_t stream);

hipError_t launch_slot_gather(const uint16_t* pool, const int32_t* idx, int64_t n, uint16_t* dst,
                              hipStream_t stream);

}  // namespace vamla
