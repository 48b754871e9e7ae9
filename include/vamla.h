/*
 * vamla.h - C ABI of libvamla: DDTree verify attention for MLA on MI355X (gfx950).
 *
 * What the library computes.  A batch of B requests; request b has a prefix of
 * L_b tokens and a drafted tree of N_b nodes (N_b <= 65).  Every token's latent
 * KV is one 576-wide bf16 row (512 latent + 64 rope) in a page_size=1 slot pool;
 * V is the first 512 columns of the same row (one latent KV head, head_dim 576).
 * For node t of request b and head h:
 *
 *   visible keys  = all L_b prefix rows  +  tree rows of t and of every ancestor of t
 *   s_l  = softmax_scale * <q[t,h,:], K_l>
 *   lse  = ln sum_l exp(s_l)              (natural log of the scaled scores)
 *   out  = sum_l exp(s_l - lse) * V_l     (rounded to bf16, nearest-even)
 *
 * Sources (web pages on DDTree verify attention):
 *   - "Mapping the Optimization Landscape for DDTree Verify Attention",
 *     "Input Knowledge Required to Understand This Message", item 1: each draft
 *     token attends only to its ancestors (read here as ancestors-or-self).
 *   - "The Architecture Detective: Uncovering FlashMLA's Potential for Blackwell
 *     DDTree Verification", "The Message in Full": the prefix is attended densely
 *     by every node with no causal constraint (causal=False, cache_seqlens=L);
 *     RoPE is applied upstream; num_heads_k=1, head_dim=576; the work splits into
 *     a dense prefix part, a small masked tree-tail part and a merge.  Here the
 *     tree tail rides along with the last prefix chunk of each request, so the
 *     split pass leaves one partial per chunk and the merge combines those.
 *   - "The Anatomy of a Kernel Investigation", "The Reasoning Process: A Deep
 *     Dive", Phase 2: the split-KV design merged through the log-sum-exp of
 *     partial attention states.
 *   - same page, "The Bash Command": page_size=1 pool with slot 0 as padding.
 *
 * Conventions for every entry point:
 *   - All tensors are row-major and densely packed.  bf16 values are passed as
 *     their 16-bit patterns (uint16_t).
 *   - Pointers marked "device" must be HIP device (or managed) memory readable
 *     by the GPU that is current when the call is made.  "host" pointers are
 *     read during the call only.
 *   - The caller owns every buffer, including the workspace.  The library never
 *     allocates or frees memory, never synchronises the stream, and keeps no
 *     pointer after returning.  All GPU work is enqueued on `stream` (a
 *     hipStream_t passed as void*; NULL = the default stream).
 *   - Return value: VAMLA_OK (0) or a negative vamla_status.  Nothing throws or
 *     aborts across the ABI.  On an error return nothing has been enqueued,
 *     except VAMLA_ERR_LAUNCH, which reports a failed kernel launch.
 *   - Contents of index arrays (slot indices in [0, pool_slots), parent arrays,
 *     cumulative lengths) are the caller's contract: the GPU path does not check
 *     them unless VAMLA_FLAG_DEBUG_VALIDATE is set.  vamla_validate checks them
 *     on host copies.
 *   - Entry points are reentrant; concurrent calls must use distinct workspaces.
 */
#ifndef VAMLA_H
#define VAMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VAMLA_D_QK 576          /* latent (512) + rope (64) */
#define VAMLA_D_V 512           /* V = columns [0, 512) of the same row */
#define VAMLA_MAX_TREE 65       /* root + up to 64 drafted nodes */
#define VAMLA_MAX_HEADS 128
#define VAMLA_KEY_TILE 32       /* chunk sizes are multiples of this */
#define VAMLA_ROW_TILE 64       /* query rows per prefix work item */

typedef enum vamla_status {
  VAMLA_OK = 0,
  VAMLA_ERR_INVALID_ARG = -1,    /* null pointer, negative size, bad flag */
  VAMLA_ERR_UNSUPPORTED = -2,    /* shape outside what the kernels handle (d_qk, d_v, H, N) */
  VAMLA_ERR_WORKSPACE = -3,      /* workspace missing or smaller than vamla_workspace_size */
  VAMLA_ERR_ARCH = -4,           /* current device is not gfx950 */
  VAMLA_ERR_LAUNCH = -5,         /* a kernel launch failed */
  VAMLA_ERR_INVALID_TREE = -6,   /* vamla_validate: parent array not topological, or not one root */
  VAMLA_ERR_INVALID_SLOT = -7,   /* vamla_validate: slot index outside [0, pool_slots) */
  VAMLA_ERR_INVALID_LENGTHS = -8, /* vamla_validate: cumulative lengths inconsistent with params */
  VAMLA_ERR_STATIC_LIMIT = -9     /* verify_attn_mla_static: the problem needs more workspace than
                                     VAMLA_STATIC_WORKSPACE_BYTES */
} vamla_status;

/*
 * Problem description shared by all verify entry points.
 *
 * Query row order: global row g = t * num_heads + h for tree node t (global
 * node index over the batch, t in [0, total_tree)) and head h.  Request b owns
 * nodes [cu_tree[b], cu_tree[b+1]) and prefix tokens [cu_prefix[b], cu_prefix[b+1])
 * of prefix_slot_idx.
 */
typedef struct vamla_params {
  int32_t batch;            /* B >= 1 */
  int32_t num_heads;        /* H in [1, 128] */
  int32_t d_qk;             /* must be 576 */
  int32_t d_v;              /* must be 512 */
  int64_t pool_slots;       /* P >= 1: rows in kv_pool */
  float softmax_scale;      /* sigma > 0 (finite), applied to q.k before the exponential */
  int32_t max_tree;         /* >= every N_b, in [1, 65] (planning bound) */
  int32_t total_tree;       /* T = cu_tree[B] >= 1; with B = 1 (and no VAMLA_FLAG_DEVICE_LENGTHS)
                               the kernels take the request's bounds from total_tree /
                               total_prefix and do not read cu_* */
  int64_t max_prefix;       /* >= every L_b (planning bound), >= 0 */
  int64_t total_prefix;     /* cu_prefix[B]; chooses the chunk size (and is L when B = 1) */
  int32_t chunk;            /* prefix keys per split; multiple of 32, or 0 = choose automatically */
  uint32_t flags;           /* 0 or an OR of VAMLA_FLAG_DEVICE_LENGTHS, VAMLA_FLAG_DEBUG_VALIDATE */
  const int32_t* cu_prefix; /* device [B+1], cu_prefix[0] = 0, non-decreasing */
  const int32_t* cu_tree;   /* device [B+1], cu_tree[0] = 0, increasing (N_b >= 1) */
  void* workspace;          /* device, 256-byte aligned, >= vamla_workspace_size bytes */
  size_t workspace_bytes;
} vamla_params;

/*
 * VAMLA_FLAG_DEVICE_LENGTHS: the kernels read every length from the device
 * arrays cu_prefix / cu_tree at run time (never from total_prefix /
 * total_tree) and choose the chunk size on the device from the longest
 * prefix they find there:
 *     chunk = max(32, 32 * ceil(ceil(Lmax / max_chunks) / 32)),
 * max_chunks being the plan's bound for max_prefix, so a request never has
 * more chunks than the plan (and the workspace) allows and a shorter prefix
 * still spreads over every chunk slot.  A captured HIP graph of a verify call
 * with this flag stays valid while the caller rewrites cu_prefix / cu_tree
 * (and the index arrays) between replays, as long as every L_b <= max_prefix,
 * every N_b <= max_tree, cu_tree[B] <= total_tree and the buffers are sized
 * for total_prefix / total_tree (the capture-time upper bounds).  Without the
 * flag a call planned for one set of lengths must be re-captured when they
 * change.  The split of a prefix into chunks can differ from the host plan's,
 * so results can differ from a call without the flag by rounding only.
 * ("The Anatomy of a Kernel Investigation", last section: the verify kernel
 * of the live service runs under CUDA-graph capture.)
 */
#define VAMLA_FLAG_DEVICE_LENGTHS 1u

/*
 * VAMLA_FLAG_DEBUG_VALIDATE: before the verify kernels, one more kernel on the
 * same stream checks on the device what vamla_validate checks on the host
 * (cumulative lengths against the params, the parent arrays, every slot index
 * against pool_slots), for callers whose index data never leaves the GPU
 * (graph capture with static buffers: "Mapping the Optimization Landscape for
 * DDTree Verify Attention", "Input Knowledge Required to Understand This
 * Message", item 5).  It writes the first violation, in the order
 * (cu arrays by request, parent by node, prefix_slot_idx by position,
 * tree_slot_idx by node), to the debug record in the workspace
 * (vamla_plan_info.off_debug_record): int32[4] = {status, array, index,
 * restarts}, status being VAMLA_ERR_INVALID_LENGTHS / _TREE / _SLOT and
 * array 0 (cu_*), 1 (parent), 2 (prefix_slot_idx) or 3 (tree_slot_idx); the
 * first three are zero when the data is valid.  restarts counts the chunk
 * restarts of the split pass (a score more than 2^96, 66.5 nats, above the
 * max of a work item's first key tile makes the item start over with a
 * higher softmax reference; see the split kernel).  When the record is set, the split kernel does no work (no
 * index is dereferenced) and the merge writes NaN to every element of out and
 * lse (total_tree x H rows).  The call itself still returns VAMLA_OK: the
 * check runs asynchronously and the caller reads the record when it syncs.
 * With vamla_lse_merge alone, the merge reads the record the preceding
 * vamla_split_partials call on the same workspace wrote.
 */
#define VAMLA_FLAG_DEBUG_VALIDATE 2u

/* Work decomposition the library derives from vamla_params (host only). */
typedef struct vamla_plan_info {
  int32_t chunk;            /* prefix keys per split (multiple of 32) */
  int32_t row_tiles;        /* ceil(max_tree * H / 64): row tiles per request */
  int32_t max_chunks;       /* ceil(max_prefix / chunk), >= 1 */
  int32_t grid_items;       /* split kernel grid (B * row_tiles * max_chunks, padded to 8) */
  /* workspace layout (byte offsets from vamla_params.workspace) */
  size_t off_part_o;        /* float [B][row_tiles][max_chunks][128 d4][64 rows][4] */
  size_t off_part_lse;      /* float [B][row_tiles][max_chunks][64 rows] */
  size_t off_debug_record;  /* int32 [4], written only with VAMLA_FLAG_DEBUG_VALIDATE */
  size_t workspace_bytes;   /* total */
} vamla_plan_info;

/*
 * Human-readable name of a status code (static string, never NULL; unknown
 * codes give "unknown status").  Host only.  Part of the error contract that
 * lets a capture-safe call report failures without throwing or aborting
 * ("Mapping the Optimization Landscape ...", "Input Knowledge Required to
 * Understand This Message", item 5).
 */
const char* vamla_status_string(int status);

/*
 * Derives the work decomposition and workspace layout.  Host only; makes no
 * HIP call, so it works without a GPU.  Returns VAMLA_ERR_INVALID_ARG or
 * VAMLA_ERR_UNSUPPORTED for parameters the kernels cannot take (among them
 * total_prefix > batch * max_prefix and total_tree > batch * max_tree).
 * Pointer fields of *p are not read; *out is written only on VAMLA_OK.  The
 * chunk split is the split-KV design of "The Anatomy of a Kernel
 * Investigation", "The Reasoning Process: A Deep Dive", Phase 2 (a dense
 * prefix in pieces, merged by log-sum-exp); the caller-owned workspace it
 * sizes is the static buffer a graph-captured call needs ("Mapping the
 * Optimization Landscape ...", "Input Knowledge ...", item 5).
 */
int vamla_plan(const vamla_params* p, vamla_plan_info* out);

/*
 * Workspace bytes verify_attn_mla needs for *p (host only, like vamla_plan;
 * *bytes is written only on VAMLA_OK).  The caller allocates it once and
 * reuses it across calls and graph replays ("Mapping the Optimization
 * Landscape ...", "Input Knowledge ...", item 5: static buffers).
 */
int vamla_workspace_size(const vamla_params* p, size_t* bytes);

/*
 * Host-side check of the index data a caller is about to pass (host copies;
 * the slot and parent conventions are those of "The Anatomy of a Kernel
 * Investigation", "The Bash Command": page_size=1 slots, and "Mapping the
 * Optimization Landscape ...", "Input Knowledge ...", item 1: each draft
 * token sees its ancestors).  Reads the host arrays only during the call:
 *   h_cu_prefix[B+1], h_cu_tree[B+1]: start at 0, prefix non-decreasing, tree
 *     increasing; totals match total_prefix / total_tree; every N_b <= max_tree,
 *     every L_b <= max_prefix;
 *   h_parent[T]: per request, parent[0] = -1 and 0 <= parent[i] < i;
 *   h_prefix_slot_idx[total_prefix], h_tree_slot_idx[T] (either may be NULL to
 *     skip): every slot in [0, pool_slots).
 * Makes no HIP call.  Returns VAMLA_OK or the first violation's code.
 */
int vamla_validate(const vamla_params* p, const int32_t* h_parent, const int32_t* h_cu_tree,
                   const int32_t* h_cu_prefix, const int32_t* h_prefix_slot_idx,
                   const int32_t* h_tree_slot_idx);

/*
 * The verify step: the split pass (prefix chunks; the last chunk of each
 * request also takes its tree keys under the ancestor mask) and the LSE merge,
 * two kernels enqueued on `stream`.  When the plan has one chunk per request
 * (vamla_plan_info.max_chunks == 1: the planner's choice for short prefixes,
 * or an explicit chunk at least max_prefix) the split pass writes out and lse
 * itself and the step is a single launch, with the same bits the two launches
 * would give (a merge of one partial multiplies it by exactly 1); the
 * workspace's partial region is then left untouched.  The pages name short
 * prefixes as where a launch-bound custom kernel lost ("The Architecture
 * Detective ...", "Context: The Performance Crisis").
 *   q               device bf16 [T, H, 576]: queries of every node (RoPE applied)
 *   kv_pool         device bf16 [P, 576]: latent rows; V = first 512 columns
 *   prefix_slot_idx device int32 [total_prefix]: pool slot of each prefix token
 *                   (may be NULL when total_prefix == 0)
 *   tree_slot_idx   device int32 [T]: pool slot of each tree node's own KV row
 *   parent          device int32 [T]: request-local parent, root = -1
 *   out             device bf16 [T, H, 512] (fully overwritten)
 *   lse             device float [T, H] (fully overwritten)
 * out and lse must not alias any input or the workspace.  Chunk boundaries are
 * fixed by logical token position, so the result does not depend on where the
 * rows sit in the pool (scrambled and contiguous pools give identical bits).
 */
int verify_attn_mla(const vamla_params* p, const uint16_t* q, const uint16_t* kv_pool,
                    const int32_t* prefix_slot_idx, const int32_t* tree_slot_idx,
                    const int32_t* parent, uint16_t* out, float* lse, void* stream);

/*
 * Stage 1 alone: split-KV attention of every row over each chunk of its
 * request's prefix, written to the workspace (part_o normalised by its own
 * softmax sum, part_lse natural log; layout in vamla_plan_info).  Chunk s of
 * request b covers prefix tokens [s*chunk, min((s+1)*chunk, L_b)); the last
 * chunk, s = max(1, ceil(L_b/chunk)) - 1, also covers the request's tree keys,
 * each row seeing the keys of its node's ancestors and itself.  Chunks past
 * that are not written.  Arguments as for verify_attn_mla.  Split-KV design:
 * "The Anatomy of a Kernel Investigation", Phase 2; the masked tree keys:
 * "Mapping the Optimization Landscape ...", "Input Knowledge Required to
 * Understand This Message", item 1.
 */
int vamla_split_partials(const vamla_params* p, const uint16_t* q, const uint16_t* kv_pool,
                         const int32_t* prefix_slot_idx, const int32_t* tree_slot_idx, const int32_t* parent,
                         void* stream);

/*
 * Stage 2 alone: merges the chunk partials in the workspace into out (bf16)
 * and lse (float): lse = ln sum_s exp(lse_s), out = sum_s exp(lse_s - lse) * o_s
 * over the max(1, ceil(L_b/chunk)) partials of each request.  Same pages:
 * merging partial attention states by their log-sum-exp.
 */
int vamla_lse_merge(const vamla_params* p, uint16_t* out, float* lse, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the verify
 * step of verify_attn_mla with the library's own workspace, a static device
 * array of VAMLA_STATIC_WORKSPACE_BYTES that each GPU holds from the first
 * such call until the process ends.  p->workspace and p->workspace_bytes are
 * ignored; everything else is as for verify_attn_mla.  The call allocates
 * nothing (no hipMalloc, no hipFree); its first call on a device looks up the
 * array's device address (hipGetSymbolAddress) and keeps it.
 * Returns VAMLA_ERR_STATIC_LIMIT, before any HIP call, when
 * vamla_workspace_size(p) exceeds the array (about 500 work items of 64
 * rows: e.g. 64k-token prefixes with 65 nodes and 16 heads need 33.5 MB).
 * Calls on one GPU share the array: calls that overlap in time on one GPU
 * (other streams, other threads) race on it and must be serialised by the
 * caller.
 */
#define VAMLA_STATIC_WORKSPACE_BYTES (64u << 20)
int verify_attn_mla_static(const vamla_params* p, const uint16_t* q, const uint16_t* kv_pool,
                           const int32_t* prefix_slot_idx, const int32_t* tree_slot_idx,
                           const int32_t* parent, uint16_t* out, float* lse, void* stream);

/*
 * Slot compaction (defragmentation) gather: dst[l, :] = kv_pool[idx[l], :] for
 * l in [0, n), bit-exact 1152-byte rows, 64-bit addressing.
 *   kv_pool device bf16 [*, 576]; idx device int32 [n] (slots must be valid);
 *   dst device bf16 [n, 576], must not overlap kv_pool rows named in idx.
 * "The Architecture Detective ...", "Defragmentation: Separating Signal from
 * Noise": compaction of scattered KV slots, secondary to the kernel itself.
 */
int vamla_slot_gather(const uint16_t* kv_pool, const int32_t* idx, int64_t n, uint16_t* dst,
                      void* stream);

/*
 * Read-rate calibration: reads the n pool rows kv_pool[idx[l], :] (1152 bytes
 * each) and does nothing with them but fold them into a checksum.  It times
 * what a plain read of exactly the rows a verify step gathers costs, the
 * practical ceiling of the split pass where it is HBM-bound (the pages
 * measure verify kernels by effective KV-read bandwidth against the HBM peak:
 * "The Anatomy of a Kernel Investigation", "Phase 3").
 *   kv_pool device bf16 [*, 576]; idx device int32 [n] (slots must be valid);
 *   sink device uint32 [VAMLA_READ_ROWS_SINK_WORDS], fully overwritten: the
 *   XOR of its words equals the XOR of every 32-bit word of the n rows (all
 *   zero for n = 0).
 * Returns VAMLA_ERR_INVALID_ARG for n < 0 or a null pointer (idx may be null
 * when n = 0).  Enqueued on stream; no allocation, no sync.
 */
#define VAMLA_READ_ROWS_SINK_WORDS 4608
int vamla_read_rows(const uint16_t* kv_pool, const int32_t* idx, int64_t n, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VAMLA_H */
