// Host side of libvamla: parameter checks, work planning, workspace layout and
// kernel launches for DDTree verify attention (see include/vamla.h).
//
// Planning, workspace sizing and validation make no HIP call, so they run on a
// host without a GPU.  The verify entry points enqueue kernels on the caller's
// stream and never allocate, free or synchronise.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>

#include "kernels.h"
#include "vamla.h"

namespace {

using namespace vamla;

static_assert(VAMLA_ROW_TILE == kRowTile, "header row tile must match the kernels");
static_assert(VAMLA_KEY_TILE == kKeyTile, "header key tile must match the kernels");
static_assert(VAMLA_D_QK == kDqk && VAMLA_D_V == kDv, "header dims must match the kernels");
static_assert(VAMLA_MAX_TREE == kMaxTree && VAMLA_MAX_HEADS == kMaxHeads, "header bounds must match the kernels");

// Chunk choice assumes the full MI355X: 256 CUs, one prefix work item per CU
// at a time (the item's key tiles fill the LDS).
constexpr int64_t kCUs = 256;
// Fixed cost of one prefix work item (loading its queries, the first key
// tiles' round trips), expressed in keys of streaming work.
constexpr int64_t kItemOverheadKeys = 256;
// Cost of one item's partial (64 rows x 2 KB written by the split pass and
// read back by the merge) at the chip's write + read rate, in the same units.
constexpr int64_t kPartialKeys = 2;
// Requests of at most 16 query rows (decode) are bound by reading the KV
// rows from HBM, and the chip serves their scattered rows faster with fewer
// concurrent streams: on the 128k-key decode step, 205 items of 640 keys ran
// 3% faster than 241 items of 544 keys, 171 items of 768 keys 2% faster and
// 128 items of 1024 keys 7% slower.  Their plans keep to this many items.
constexpr int64_t kHbmBoundItems = 208;
// What the merge launch costs a short step beyond the work it takes off the
// split pass, in keys of streaming work.  A plan with one chunk per request
// skips it: the split pass writes the output itself.  Fitted to the measured
// crossover on 9- and 65-node trees of 16 heads: one launch is faster at
// 64-key prefixes (14.4 against 15.1 us, 16.9 against 18.3 us), ties at 128
// keys with 65 nodes and is slower from 128 keys with 9 nodes (16.4 against
// 15.3 us), which bounds this cost to 20..72 keys.
constexpr int64_t kMergeKeys = 48;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_shape(const vamla_params* p) {
  if (!p) return VAMLA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->pool_slots < 1 || p->max_prefix < 0 || p->total_prefix < 0 || p->total_tree < 1)
    return VAMLA_ERR_INVALID_ARG;
  if ((p->flags & ~(VAMLA_FLAG_DEVICE_LENGTHS | VAMLA_FLAG_DEBUG_VALIDATE)) != 0) return VAMLA_ERR_INVALID_ARG;
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f)) return VAMLA_ERR_INVALID_ARG;
  if (p->d_qk != VAMLA_D_QK || p->d_v != VAMLA_D_V) return VAMLA_ERR_UNSUPPORTED;
  if (p->num_heads < 1 || p->num_heads > VAMLA_MAX_HEADS) return VAMLA_ERR_UNSUPPORTED;
  if (p->max_tree < 1 || p->max_tree > VAMLA_MAX_TREE) return VAMLA_ERR_UNSUPPORTED;
  if (p->chunk < 0 || p->chunk % VAMLA_KEY_TILE != 0) return VAMLA_ERR_INVALID_ARG;
  // 32-bit index arithmetic inside the kernels
  if (p->max_prefix > (int64_t)INT32_MAX - 2 * VAMLA_KEY_TILE || p->total_prefix > (int64_t)INT32_MAX)
    return VAMLA_ERR_UNSUPPORTED;
  if ((int64_t)p->total_tree * p->num_heads > (int64_t)INT32_MAX / VAMLA_D_V) return VAMLA_ERR_UNSUPPORTED;
  if (p->pool_slots > (int64_t)UINT32_MAX) return VAMLA_ERR_UNSUPPORTED;
  // the totals must fit the planning bounds: chunks and row tiles are sized
  // from max_prefix / max_tree, so a longer request would be cut short
  if (p->total_prefix > (int64_t)p->batch * p->max_prefix) return VAMLA_ERR_INVALID_ARG;
  if ((int64_t)p->total_tree > (int64_t)p->batch * p->max_tree) return VAMLA_ERR_INVALID_ARG;
  return VAMLA_OK;
}

int64_t choose_chunk(const vamla_params* p, int64_t row_tiles, int64_t rows) {
  if (p->chunk > 0) return p->chunk;
  const int64_t maxL = p->max_prefix;
  if (maxL <= VAMLA_KEY_TILE) return VAMLA_KEY_TILE;
  const int64_t total = p->total_prefix > 0 ? p->total_prefix : maxL;
  // the last chunk of a request also streams its tree keys (whole tiles)
  const int64_t tree_keys = ceil_div(p->max_tree, VAMLA_KEY_TILE) * VAMLA_KEY_TILE;
  // Candidates: the longest prefix split into k chunks, k = 1, 2, ...; cost =
  // rounds of work items over the CUs times the keys the largest item
  // streams, plus the partials' traffic (which makes small problems prefer
  // fewer, longer chunks).  The cost depends on the chunk size c(k) only, so
  // the loop visits each distinct c once: after c, the next smaller size
  // needs ceil(maxL / k) <= c - tile, i.e. k >= ceil(maxL / (c - tile)).
  int64_t best_c = VAMLA_KEY_TILE, best_cost = INT64_MAX;
  const int64_t kmax = std::min<int64_t>(ceil_div(maxL, VAMLA_KEY_TILE), 8192);
  for (int64_t k = 1, c = 0; k <= kmax; k = (c > VAMLA_KEY_TILE) ? ceil_div(maxL, c - VAMLA_KEY_TILE) : kmax + 1) {
    c = ceil_div(ceil_div(maxL, k), VAMLA_KEY_TILE) * VAMLA_KEY_TILE;
    // each request contributes its full chunks plus at most one partial one;
    // only the lengths' sum and maximum are known here, and a request's
    // last chunk is half full on average, so the partial ones add about B/2
    const int64_t chunks =
        std::min<int64_t>(ceil_div(total, c) + ceil_div(p->batch - 1, 2), (int64_t)p->batch * ceil_div(maxL, c));
    const int64_t items = row_tiles * chunks;
    // HBM-bound plans skip chunk sizes with more items than the knee (the
    // largest candidate, one chunk per request, always stays)
    if (rows <= 16 && items > kHbmBoundItems && k > 1) continue;
    const int64_t rounds = ceil_div(items, kCUs);
    const int64_t last = maxL - (ceil_div(maxL, c) - 1) * c;
    const int64_t item_keys = std::max(c, ceil_div(last, VAMLA_KEY_TILE) * VAMLA_KEY_TILE + tree_keys);
    const int64_t cost =
        rounds * (item_keys + kItemOverheadKeys) + (c >= maxL ? 0 : items * kPartialKeys + kMergeKeys);
    if (cost < best_cost || (cost == best_cost && c > best_c)) {   // ties: larger chunk, fewer partials
      best_cost = cost;
      best_c = c;
    }
  }
  return best_c;
}

// The plan depends only on the scalar fields of the parameters, so a caller
// that repeats one shape (a serving loop) gets it from a cache: one entry per
// host thread, so concurrent callers never share it.
struct PlanKey {
  int32_t batch, num_heads, d_qk, d_v;
  int64_t pool_slots;
  float softmax_scale;
  int32_t max_tree, total_tree;
  int64_t max_prefix, total_prefix;
  int32_t chunk;
  uint32_t flags;
};
thread_local PlanKey t_plan_key;
thread_local vamla_plan_info t_plan;
thread_local bool t_plan_valid = false;

int make_plan_uncached(const vamla_params* p, vamla_plan_info* out);

int make_plan(const vamla_params* p, vamla_plan_info* out) {
  if (!p) return VAMLA_ERR_INVALID_ARG;
  PlanKey k;
  std::memset(&k, 0, sizeof(k));   // padding included, for the byte compare
  k.batch = p->batch;
  k.num_heads = p->num_heads;
  k.d_qk = p->d_qk;
  k.d_v = p->d_v;
  k.pool_slots = p->pool_slots;
  k.softmax_scale = p->softmax_scale;
  k.max_tree = p->max_tree;
  k.total_tree = p->total_tree;
  k.max_prefix = p->max_prefix;
  k.total_prefix = p->total_prefix;
  k.chunk = p->chunk;
  k.flags = p->flags;
  if (t_plan_valid && std::memcmp(&k, &t_plan_key, sizeof(k)) == 0) {
    *out = t_plan;
    return VAMLA_OK;
  }
  const int st = make_plan_uncached(p, out);
  if (st == VAMLA_OK) {
    t_plan_key = k;
    t_plan = *out;
    t_plan_valid = true;
  }
  return st;
}

int make_plan_uncached(const vamla_params* p, vamla_plan_info* out) {
  const int st = check_shape(p);
  if (st != VAMLA_OK) return st;
  vamla_plan_info pl;
  std::memset(&pl, 0, sizeof(pl));
  const int64_t rows = (int64_t)p->max_tree * p->num_heads;
  const int64_t row_tiles = ceil_div(rows, kRowTile);
  const int64_t chunk = choose_chunk(p, row_tiles, rows);
  const int64_t max_chunks = std::max<int64_t>(1, ceil_div(p->max_prefix, chunk));
  const int64_t items = (int64_t)p->batch * row_tiles * max_chunks;
  if (items > (int64_t)INT32_MAX / 2) return VAMLA_ERR_UNSUPPORTED;
  pl.chunk = (int32_t)chunk;
  pl.row_tiles = (int32_t)row_tiles;
  pl.max_chunks = (int32_t)max_chunks;
  pl.grid_items = (int32_t)(ceil_div(items, 8) * 8);
  const size_t item_o = (size_t)kD4 * kRowTile * 4 * sizeof(float);
  const size_t item_l = (size_t)kRowTile * sizeof(float);
  size_t off = 0;
  pl.off_part_o = off;
  off = align256(off + (size_t)items * item_o);
  pl.off_part_lse = off;
  off = align256(off + (size_t)items * item_l);
  pl.off_debug_record = off;
  off = align256(off + 4 * sizeof(int32_t));
  pl.workspace_bytes = off;
  *out = pl;
  return VAMLA_OK;
}

std::atomic<int> g_arch_state[64];   // 0 unknown, 1 gfx950, -1 other

int check_arch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VAMLA_ERR_ARCH;
  if (dev < 0 || dev >= 64) return VAMLA_ERR_ARCH;
  int s = g_arch_state[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return VAMLA_ERR_ARCH;
    s = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_arch_state[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? VAMLA_OK : VAMLA_ERR_ARCH;
}

int workspace_ok(const vamla_params* p, const vamla_plan_info& pl) {
  if (!p->workspace || p->workspace_bytes < pl.workspace_bytes) return VAMLA_ERR_WORKSPACE;
  if (((uintptr_t)p->workspace & 255) != 0) return VAMLA_ERR_WORKSPACE;
  return VAMLA_OK;
}

float* ws_f(const vamla_params* p, size_t off) { return (float*)((char*)p->workspace + off); }

int32_t* debug_record(const vamla_params* p, const vamla_plan_info& pl) {
  return (p->flags & VAMLA_FLAG_DEBUG_VALIDATE) ? (int32_t*)((char*)p->workspace + pl.off_debug_record) : nullptr;
}

int validate_launch(const vamla_params* p, const vamla_plan_info& pl, const int32_t* prefix_slot_idx,
                    const int32_t* tree_slot_idx, const int32_t* parent, hipStream_t stream) {
  ValidateArgs a;
  a.cu_prefix = p->cu_prefix;
  a.cu_tree = p->cu_tree;
  a.parent = parent;
  a.prefix_slot = prefix_slot_idx;
  a.tree_slot = tree_slot_idx;
  a.record = debug_record(p, pl);
  a.max_prefix = p->max_prefix;
  a.total_prefix = p->total_prefix;
  a.pool_slots = p->pool_slots;
  a.batch = p->batch;
  a.max_tree = p->max_tree;
  a.total_tree = p->total_tree;
  a.device_lengths = (p->flags & VAMLA_FLAG_DEVICE_LENGTHS) ? 1 : 0;
  return launch_debug_validate(a, stream) == hipSuccess ? VAMLA_OK : VAMLA_ERR_LAUNCH;
}

int split_launch(const vamla_params* p, const vamla_plan_info& pl, const uint16_t* q, const uint16_t* pool,
                 const int32_t* prefix_slot_idx, const int32_t* tree_slot_idx, const int32_t* parent,
                 uint16_t* out, float* lse, hipStream_t stream) {
  PrefixArgs a;
  a.q = q;
  a.pool = pool;
  a.prefix_slot = prefix_slot_idx;
  a.tree_slot = tree_slot_idx;
  a.parent = parent;
  a.cu_prefix = p->cu_prefix;
  a.cu_tree = p->cu_tree;
  a.part_o = ws_f(p, pl.off_part_o);
  a.part_lse = ws_f(p, pl.off_part_lse);
  a.num_heads = p->num_heads;
  a.chunk = pl.chunk;
  a.row_tiles = pl.row_tiles;
  a.max_chunks = pl.max_chunks;
  a.batch = p->batch;
  a.grid_items = pl.grid_items;
  a.total_prefix = (int32_t)p->total_prefix;
  a.total_tree = p->total_tree;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.device_lengths = (p->flags & VAMLA_FLAG_DEVICE_LENGTHS) ? 1 : 0;
  a.debug_record = debug_record(p, pl);
  a.out = out;
  a.lse = lse;
  if (a.debug_record) {
    const int st = validate_launch(p, pl, prefix_slot_idx, tree_slot_idx, parent, stream);
    if (st != VAMLA_OK) return st;
  }
  return launch_prefix_splitkv(a, stream) == hipSuccess ? VAMLA_OK : VAMLA_ERR_LAUNCH;
}

int merge_launch(const vamla_params* p, const vamla_plan_info& pl, uint16_t* out, float* lse, hipStream_t stream) {
  MergeArgs a;
  a.part_o = ws_f(p, pl.off_part_o);
  a.part_lse = ws_f(p, pl.off_part_lse);
  a.cu_prefix = p->cu_prefix;
  a.cu_tree = p->cu_tree;
  a.out = out;
  a.lse = lse;
  a.num_heads = p->num_heads;
  a.chunk = pl.chunk;
  a.row_tiles = pl.row_tiles;
  a.max_chunks = pl.max_chunks;
  a.batch = p->batch;
  a.total_prefix = (int32_t)p->total_prefix;
  a.total_tree = p->total_tree;
  a.device_lengths = (p->flags & VAMLA_FLAG_DEVICE_LENGTHS) ? 1 : 0;
  a.debug_record = debug_record(p, pl);
  // a wave covers the live rows of a tile (at most max_tree * H when there is
  // one row tile), its other lanes split the chunks
  const int64_t tile_rows = std::min<int64_t>(kRowTile, (int64_t)p->max_tree * p->num_heads);
  int bits = 0;
  while ((1 << bits) < tile_rows) ++bits;
  a.row_bits = bits;
  // waves per column group that split its chunks: one when the grid has
  // >= 512 workgroups (2 per CU) or when one thread's chunks fit in one batch
  // of loads (16); otherwise the fewest that bring a thread's share of the
  // chunks to one batch (at most 4).  Splitting costs an exchange through
  // LDS, so it pays only where it removes a round trip.
  const int64_t base = (int64_t)p->batch * pl.row_tiles * (kD4 / 4);
  const int64_t lanes_per_row = 64 >> bits;   // chunk lanes of a wave
  auto batches = [&](int cw) { return ceil_div(ceil_div(pl.max_chunks, lanes_per_row << cw), 16); };
  int cw_bits = 0;
  if (base < 512 && batches(0) > 1) cw_bits = batches(1) == 1 ? 1 : 2;
  a.chunk_wave_bits = cw_bits;
  return launch_lse_merge(a, stream) == hipSuccess ? VAMLA_OK : VAMLA_ERR_LAUNCH;
}

// Common checks of every verify-family entry point; fills the plan.
int prologue(const vamla_params* p, vamla_plan_info* pl) {
  int st = make_plan(p, pl);
  if (st != VAMLA_OK) return st;
  if (!p->cu_prefix || !p->cu_tree) return VAMLA_ERR_INVALID_ARG;
  st = workspace_ok(p, *pl);
  if (st != VAMLA_OK) return st;
  return check_arch();
}

}  // namespace

extern "C" {

const char* vamla_status_string(int status) {
  switch (status) {
    case VAMLA_OK: return "ok";
    case VAMLA_ERR_INVALID_ARG: return "invalid argument";
    case VAMLA_ERR_UNSUPPORTED: return "unsupported shape";
    case VAMLA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case VAMLA_ERR_ARCH: return "current device is not gfx950";
    case VAMLA_ERR_LAUNCH: return "kernel launch failed";
    case VAMLA_ERR_INVALID_TREE: return "invalid tree (parent array)";
    case VAMLA_ERR_INVALID_SLOT: return "slot index out of range";
    case VAMLA_ERR_INVALID_LENGTHS: return "cumulative lengths inconsistent";
    case VAMLA_ERR_STATIC_LIMIT: return "problem needs more workspace than the static workspace holds";
    default: return "unknown status";
  }
}

int vamla_plan(const vamla_params* p, vamla_plan_info* out) {
  if (!out) return VAMLA_ERR_INVALID_ARG;
  return make_plan(p, out);
}

int vamla_workspace_size(const vamla_params* p, size_t* bytes) {
  if (!bytes) return VAMLA_ERR_INVALID_ARG;
  vamla_plan_info pl;
  const int st = make_plan(p, &pl);
  if (st != VAMLA_OK) return st;
  *bytes = pl.workspace_bytes;
  return VAMLA_OK;
}

int vamla_validate(const vamla_params* p, const int32_t* h_parent, const int32_t* h_cu_tree,
                   const int32_t* h_cu_prefix, const int32_t* h_prefix_slot_idx,
                   const int32_t* h_tree_slot_idx) {
  int st = check_shape(p);
  if (st != VAMLA_OK) return st;
  if (!h_parent || !h_cu_tree || !h_cu_prefix) return VAMLA_ERR_INVALID_ARG;
  if (h_cu_tree[0] != 0 || h_cu_prefix[0] != 0) return VAMLA_ERR_INVALID_LENGTHS;
  for (int b = 0; b < p->batch; ++b) {
    const int64_t n = (int64_t)h_cu_tree[b + 1] - h_cu_tree[b];
    const int64_t l = (int64_t)h_cu_prefix[b + 1] - h_cu_prefix[b];
    if (n < 1 || n > p->max_tree) return VAMLA_ERR_INVALID_LENGTHS;
    if (l < 0 || l > p->max_prefix) return VAMLA_ERR_INVALID_LENGTHS;
  }
  if (h_cu_tree[p->batch] != p->total_tree) return VAMLA_ERR_INVALID_LENGTHS;
  if (h_cu_prefix[p->batch] != p->total_prefix) return VAMLA_ERR_INVALID_LENGTHS;
  for (int b = 0; b < p->batch; ++b) {
    const int t0 = h_cu_tree[b], n = h_cu_tree[b + 1] - t0;
    if (h_parent[t0] != -1) return VAMLA_ERR_INVALID_TREE;
    for (int i = 1; i < n; ++i) {
      const int pa = h_parent[t0 + i];
      if (pa < 0 || pa >= i) return VAMLA_ERR_INVALID_TREE;
    }
  }
  if (h_prefix_slot_idx) {
    for (int64_t i = 0; i < p->total_prefix; ++i)
      if (h_prefix_slot_idx[i] < 0 || h_prefix_slot_idx[i] >= p->pool_slots) return VAMLA_ERR_INVALID_SLOT;
  }
  if (h_tree_slot_idx) {
    for (int64_t i = 0; i < p->total_tree; ++i)
      if (h_tree_slot_idx[i] < 0 || h_tree_slot_idx[i] >= p->pool_slots) return VAMLA_ERR_INVALID_SLOT;
  }
  return VAMLA_OK;
}

int verify_attn_mla(const vamla_params* p, const uint16_t* q, const uint16_t* kv_pool,
                    const int32_t* prefix_slot_idx, const int32_t* tree_slot_idx, const int32_t* parent,
                    uint16_t* out, float* lse, void* stream) {
  vamla_plan_info pl;
  int st = prologue(p, &pl);
  if (st != VAMLA_OK) return st;
  if (!q || !kv_pool || !tree_slot_idx || !parent || !out || !lse) return VAMLA_ERR_INVALID_ARG;
  if (p->total_prefix > 0 && !prefix_slot_idx) return VAMLA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  // one chunk per request: the split pass writes out and lse itself and the
  // step is a single launch (the merge of one partial is the identity)
  if (pl.max_chunks == 1) return split_launch(p, pl, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, out, lse, s);
  st = split_launch(p, pl, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, nullptr, nullptr, s);
  if (st != VAMLA_OK) return st;
  return merge_launch(p, pl, out, lse, s);
}

int vamla_split_partials(const vamla_params* p, const uint16_t* q, const uint16_t* kv_pool,
                         const int32_t* prefix_slot_idx, const int32_t* tree_slot_idx, const int32_t* parent,
                         void* stream) {
  vamla_plan_info pl;
  int st = prologue(p, &pl);
  if (st != VAMLA_OK) return st;
  if (!q || !kv_pool || !tree_slot_idx || !parent) return VAMLA_ERR_INVALID_ARG;
  if (p->total_prefix > 0 && !prefix_slot_idx) return VAMLA_ERR_INVALID_ARG;
  return split_launch(p, pl, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, nullptr, nullptr,
                      (hipStream_t)stream);
}

int vamla_lse_merge(const vamla_params* p, uint16_t* out, float* lse, void* stream) {
  vamla_plan_info pl;
  int st = prologue(p, &pl);
  if (st != VAMLA_OK) return st;
  if (!out || !lse) return VAMLA_ERR_INVALID_ARG;
  return merge_launch(p, pl, out, lse, (hipStream_t)stream);
}

int vamla_slot_gather(const uint16_t* kv_pool, const int32_t* idx, int64_t n, uint16_t* dst, void* stream) {
  if (n < 0) return VAMLA_ERR_INVALID_ARG;
  if (n == 0) return VAMLA_OK;
  if (!kv_pool || !idx || !dst) return VAMLA_ERR_INVALID_ARG;
  const int st = check_arch();
  if (st != VAMLA_OK) return st;
  return launch_slot_gather(kv_pool, idx, n, dst, (hipStream_t)stream) == hipSuccess ? VAMLA_OK
                                                                                     : VAMLA_ERR_LAUNCH;
}

int vamla_read_rows(const uint16_t* kv_pool, const int32_t* idx, int64_t n, uint32_t* sink, void* stream) {
  if (n < 0 || !kv_pool || !sink || (n > 0 && !idx)) return VAMLA_ERR_INVALID_ARG;
  const int st = check_arch();
  if (st != VAMLA_OK) return st;
  return launch_read_rows(kv_pool, idx, n, sink, (hipStream_t)stream) == hipSuccess ? VAMLA_OK : VAMLA_ERR_LAUNCH;
}

}  // extern "C"
