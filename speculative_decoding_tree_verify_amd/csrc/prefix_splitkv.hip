// Split-KV pass of DDTree verify attention over an MLA latent pool (gfx950).
//
// Every tree node attends densely to the whole prefix with no mask ("The
// Architecture Detective: Uncovering FlashMLA's Potential for Blackwell DDTree
// Verification", "The Message in Full": causal=False over the prefix, one
// latent head of width 576 whose first 512 columns are V).  The prefix is cut
// into fixed chunks of logical positions; each chunk yields a normalised
// partial (o_s, lse_s) that a later pass merges by log-sum-exp ("The Anatomy of
// a Kernel Investigation", "The Reasoning Process: A Deep Dive", Phase 2).  The
// last chunk of a request also takes the request's tree keys, each row seeing
// only its node's ancestors and itself ("Mapping the Optimization Landscape
// for DDTree Verify Attention", "Input Knowledge Required to Understand This
// Message", item 1), so one partial covers both.
//
// Work item = (request b, row tile of 64 query rows, chunk s); one 512-thread
// workgroup per item, two waves per SIMD, specialised:
//   * 4 QK waves.  Wave w holds all 576 query columns of 32 rows (rows
//     32(w>>1) ..) in VGPRs and, per 32-key tile, computes the scores of its 16
//     keys (keys 16(w&1) ..): S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K
//     from LDS, B = Q; each K fragment feeds both 16-row halves).  It then
//     forms P = exp2(S*scale*log2e - m) in bf16 and stores it to LDS in the PV
//     waves' operand layout.
//   * 4 PV waves.  Wave c accumulates O^T += V^T P^T for output columns
//     [128c, 128c+128) of all 64 rows with v_mfma_f32_32x32x16_bf16 (A = V^T
//     read by ds_read_b64_tr_b16, B = P; each V^T fragment feeds both row
//     halves), 128 accumulator VGPRs, and issues the gather of the tiles ahead.
// The SIMD's matrix core is shared by its QK and PV wave, so one wave's
// softmax, LDS waits and gather issue overlap the other's MFMAs.  One barrier
// per tile and a three-stage pipeline: in iteration t the QK waves score tile
// t and turn the scores of tile t-1 into P(t-1) (that softmax runs while tile
// t's first K fragments are in flight); the PV waves multiply V(t-2), read
// into VGPRs during iteration t-1, by P(t-2), read V(t-1) fragment by
// fragment as the registers free up, and gather tile t+2 once their first
// four MFMAs are under way.  The restart vote of tile t-2 is read early and
// tested just before the barrier.  A tile whose query rows end inside it
// skips the Q loads and MFMAs of its dead 16-row halves (QK; with no live
// row in a pair, its K reads too) and the MFMAs of rows 32..63 (PV) when
// they hold no live row.  A tile of more than 16 live rows brings its query
// rows to the QK waves' registers through LDS: contiguous LDS-DMA into the
// two ring slots the loop fills last, then fragment reads.
// With the request lengths read on the device, the chunk size comes from
// the longest prefix in cu_prefix (device_chunk) instead of the host plan.
//
// Gather: LDS-DMA moves 16 bytes per lane straight into LDS.  PV wave c
// gathers keys 8c .. 8c+7 of a tile with nine 64-lane global_load_lds_dwordx4,
// one per 128-byte column group of the rows (8 latent groups, then the rope);
// every lane keeps one 64-bit address (its key's row plus its piece, so rows
// may lie past 4 GiB) and the instruction offset steps it from group to group
// (the offset moves the LDS destination as well, so M0 advances by the rest
// of a group).  The DMAs are asm: the compiler would otherwise make every LDS
// read wait for them (it cannot tell the ring slots apart); the waits are
// explicit vmcnt counts before each barrier.  The PV waves' LDS reads are asm
// too, with lgkmcnt waits counted by hand, so that the V reads of the next
// tile stay in flight under the current tile's MFMAs.  A 4-slot ring of 36 KB
// tiles (32 keys), each four 9 KB units of 8 keys (the unit a wave gathers):
//   unit u = key >> 3 at u*9216; group d (pieces 8d .. 8d+7 of the 8 keys) at
//   +1024d; key k8 = key & 7 at +128 k8; piece p of the group at slot
//   p ^ swz(k8), swz(k8) = ((k8 & 2) << 1) | ((k8 & 4) >> 1) | (k8 & 1).
// The QK ds_read_b128 pattern (8 consecutive keys at one piece per LDS cycle)
// hits 8 distinct slots because swz is a permutation; the PV
// ds_read_b64_tr_b16 pattern (4 keys x 4 pieces x 2 halves per 32 lanes)
// covers all 64 banks because swz(k8) ^ swz(k8 + 2) has bit 2 set for the
// key pairs that share a bank half.  A lane's K fragment of step st is at a
// fixed base ^ 64(st & 1) + 1024(st >> 1); its V^T fragment (4ks + cb) at a
// fixed base ^ 64(cb & 1) + 18432 ks + 1024(cb >> 1).

// Softmax reference: each row keeps a reference m (log2 units) instead of a
// running max, so the accumulators are never rescaled.  The first tile sets m
// to the row's max over that tile plus kMargin (the two QK waves of a row pair
// exchange their halves through LDS at the first barrier).  While every score
// stays within kSlack of m, exp2(s - m) <= 2^kSlack, inside bf16/fp32 range
// (the accumulators overflow only if |V| * keys of a chunk reached
// 2^(128 - kSlack)); the row's own max term is at least 2^-kMargin, so its sum
// stays far from underflow, and only terms below 2^-126, under 2^-(126 -
// kMargin) of the max term, can flush.  A tile that breaks this (a score more than kMargin + kSlack
// = 96 log2 units, 66.5 nats, above the first tile's max: rare) makes the
// workgroup restart its item with each row's m raised to max(m, the row's max
// over that tile + kMargin).  Every m stays at or below the row's true max +
// kMargin, so no row's exponentials drift towards underflow however many
// restarts there are; each restart needs a new tile max more than kSlack above
// a reference and leaves every row's m above that tile's max, so there are at
// most as many restarts as tiles.  With the debug flag the kernel adds its
// restarts to a counter in the debug record.

#include "kernels.h"

namespace vamla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kSlack = 56.0f;               // headroom above the reference (log2)
constexpr float kMargin = 40.0f;              // reference above the first tile's max (log2)
constexpr int kKT = 32;                       // keys per tile
constexpr int kTileLds = kKT * kDqk * 2;      // 36864 B
constexpr int kUnit = 8 * kDqk * 2;            // 9216 B: the 8 keys one wave gathers
constexpr int kGroup = 1024;                  // 16-byte pieces 8d .. 8d+7 of the unit's 8 keys
// LDS-DMA M0 step between the nine DMAs of a gather, which share one address
// register and advance their source with the instruction offset (128 B per
// group); the offset also moves the LDS destination, so M0 advances by the
// rest of a group
constexpr int kM0Step = kGroup - 128;
constexpr int kRing = 4;                      // tiles staged in LDS
constexpr int kQSteps = kDqk / 32;            // 18 steps of v_mfma_f32_16x16x32_bf16
constexpr int kPreQK = 4;                     // K fragments read ahead
constexpr int kCompactBatch = 64;             // requests scanned per workgroup to list real items

// slot of piece p (0..7) of key k8 (0..7) inside a group: p ^ swz(k8)
__device__ __forceinline__ int swz(int k8) { return ((k8 & 2) << 1) | ((k8 & 4) >> 1) | (k8 & 1); }

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A 4-byte global load issued as asm: its result is valid only after an
// explicit vmcnt wait that names the register.
__device__ __forceinline__ uint32_t load_u32_async(const int* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}


// LDS reads issued as asm: the compiler does not count them, so each use is
// preceded by an explicit lgkmcnt wait that names the register.  LDS
// operations of one wave complete in order, so lgkmcnt(n) means "all but the
// last n issued LDS operations have landed".
#define VAMLA_LGKM_CASE(N) case N: asm volatile("s_waitcnt lgkmcnt(" #N ")" : "+v"(r) :: "memory"); break;
template <typename T>
__device__ __forceinline__ void wait_lgkm(int n, T& r) {
  switch (n) {
    VAMLA_LGKM_CASE(0) VAMLA_LGKM_CASE(1) VAMLA_LGKM_CASE(2) VAMLA_LGKM_CASE(3) VAMLA_LGKM_CASE(4)
    VAMLA_LGKM_CASE(5) VAMLA_LGKM_CASE(6) VAMLA_LGKM_CASE(7) VAMLA_LGKM_CASE(8) VAMLA_LGKM_CASE(9)
    VAMLA_LGKM_CASE(10) VAMLA_LGKM_CASE(11) VAMLA_LGKM_CASE(12) VAMLA_LGKM_CASE(13) VAMLA_LGKM_CASE(14)
    default: asm volatile("s_waitcnt lgkmcnt(15)" : "+v"(r) :: "memory"); break;
  }
}
#undef VAMLA_LGKM_CASE
#define VAMLA_B128_CASE(O) case O: asm volatile("ds_read_b128 %0, %1 offset:" #O : "=v"(v) : "v"(addr)); break;
__device__ __forceinline__ bf16x8 ds_b128(uint32_t addr, int off) {
  bf16x8 v;
  switch (off) {
    VAMLA_B128_CASE(0) VAMLA_B128_CASE(1024) VAMLA_B128_CASE(2048) VAMLA_B128_CASE(3072)
    default: __builtin_trap();
  }
  return v;
}
#undef VAMLA_B128_CASE
#define VAMLA_TR_CASE(O) case O: asm volatile("ds_read_b64_tr_b16 %0, %1 offset:" #O : "=v"(v) : "v"(addr)); break;
__device__ __forceinline__ i16x4 ds_tr(uint32_t addr, int off) {
  i16x4 v;
  switch (off) {
    VAMLA_TR_CASE(0) VAMLA_TR_CASE(1024) VAMLA_TR_CASE(18432) VAMLA_TR_CASE(19456)
    default: __builtin_trap();
  }
  return v;
}
#undef VAMLA_TR_CASE
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }

// max without the NaN-quieting the compiler adds around fmaxf (scores are
// never signalling NaNs here; -inf marks masked keys)
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ void swap32(float& p, float& q) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(p), "+v"(q));
}
__device__ __forceinline__ void swap16(float& p, float& q) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(p), "+v"(q));
}
// sum of x over the four lanes l % 16 == const
__device__ __forceinline__ float sum4(float x) {
  float p = x, q = x;
  swap16(p, q);
  float y = p + q;
  p = y;
  q = y;
  swap32(p, q);
  return p + q;
}

// The nine LDS-DMAs that gather PV wave c's 8 keys of a 32-key tile (keys
// 8c .. 8c+7, unit c of the tile).  Lane l moves, for group d = 0..8, the
// 16-byte piece 8d + ((l & 7) ^ swz(l >> 3)) of key 8c + (l >> 3) into LDS at
// unit + 1024 d + 16 l, i.e. to slot l & 7 of that key's 128 bytes of the
// group.  One 64-bit address per lane (its key's row plus its piece) serves
// all nine: the instruction offset steps the source by 128 B per group.
// sv: slot index of key 8c + (lane >> 3); pool_lane: pool + this lane's
// piece offset.
__device__ __forceinline__ void gather_tile(const uint8_t* pool_lane, uint32_t sv, uint8_t* buf, int c) {
  const uint8_t* src = pool_lane + (size_t)sv * (kDqk * 2);
  const uint32_t m = (uint32_t)(uintptr_t)(lds_void*)(buf + c * kUnit);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:128\n\t"
      "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:256\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:384\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:512\n\t"
      "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:640\n\t"
      "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:768\n\t"
      "s_mov_b32 m0, %9\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:896\n\t"
      "s_mov_b32 m0, %10\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:1024\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(m), "s"(m + 1 * kM0Step), "s"(m + 2 * kM0Step), "s"(m + 3 * kM0Step), "s"(m + 4 * kM0Step),
        "s"(m + 5 * kM0Step), "s"(m + 6 * kM0Step), "s"(m + 7 * kM0Step), "s"(m + 8 * kM0Step)
      : "memory");
}

// One LDS-DMA: lane l's 16 bytes at src go to LDS m + 16 l (m uniform).
__device__ __forceinline__ void dma_1k(const void* src, uint32_t m) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(src), "s"(m)
               : "memory");
}

// Query rows staged in LDS for the QK waves' registers: the 32 rows of a
// pair (36 KB, contiguous in q) sit row-major, 72 pieces of 16 bytes a row,
// piece p of row r at slot p ^ qswz(r).  The DMAs then copy contiguous
// kilobytes of q, and the fragment reads (16 rows at one piece) hit 16
// distinct bank quads: row r's quad is 8(r & 1) + the slot's low bits.
__device__ __forceinline__ int qswz(int r) { return (r >> 1) & 7; }

struct Shared {
  uint8_t pbuf[2][4][1024];                   // P operands, [parity][ks*2 + rb][lane*16]
  float2 mtl[3][4][64];                       // QK waves: per-lane max of each 16-row half, by tile mod 3
  float want[2][4];                           // QK waves: restart vote per tile parity
  float rowl[64];                             // final row sums (QK -> PV)
  uint32_t vis[kRowTile][4];                  // tree masks: bit k of word tt = tree key 32tt + k visible
  int par[kMaxTree];
};

__global__ __launch_bounds__(512, 1) void prefix_splitkv_kernel(PrefixArgs a) {
  // Four staged tiles as separate arrays: the PV loop names each one
  // statically, so the compiler can tell a gather's destination from the
  // tile being read and does not drain the gathers before every LDS read.
  __shared__ __attribute__((aligned(1024))) uint8_t tile0[kTileLds];
  __shared__ __attribute__((aligned(1024))) uint8_t tile1[kTileLds];
  __shared__ __attribute__((aligned(1024))) uint8_t tile2[kTileLds];
  __shared__ __attribute__((aligned(1024))) uint8_t tile3[kTileLds];
  __shared__ __attribute__((aligned(16))) Shared sh;
  static_assert(kRing == 4, "ring slots are picked by the low two bits of the tile index");
  auto ring = [&](int i) -> uint8_t* { i &= kRing - 1; return i == 0 ? tile0 : i == 1 ? tile1 : i == 2 ? tile2 : tile3; };

  // The arguments that the item decode and the first loads need are named
  // here, so that every kernel-argument load is issued at once: left to the
  // compiler, those behind the debug test below wait for its loads, a second
  // dependent round trip before the first slot index can be read.
  asm volatile("" ::"s"(a.q), "s"(a.prefix_slot), "s"(a.tree_slot), "s"(a.cu_prefix), "s"(a.part_lse),
               "s"(a.device_lengths), "s"(a.scale_log2));
  // with the debug flag, a failed device-side index check leaves no work;
  // when this pass writes the final output (one chunk per request), every
  // element of it is NaN instead, as the merge would make it
  if (a.debug_record && __builtin_amdgcn_readfirstlane(a.debug_record[0]) != 0) {
    if (a.out) {
      const int64_t rows = (int64_t)a.total_tree * a.num_heads;
      const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
      const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
      const uint2 nan2 = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
      for (int64_t i = gid; i < rows * (kDv / 4); i += nthreads) *(uint2*)(a.out + i * 4) = nan2;
      for (int64_t i = gid; i < rows; i += nthreads) a.lse[i] = __builtin_nanf("");
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool is_qk = w < 4;

  // Work item -> (request b, chunk s, row tile).  Real items are listed in
  // request order, a chunk's row tiles consecutive; XCD x (= blockIdx % 8,
  // the round-robin dispatch) takes the x-th contiguous eighth of the list,
  // so the row tiles of a chunk share an XCD's L2 and every XCD gets the same
  // number of items however unequal the requests are.  Requests with no tree
  // node have no items.  Past kCompactBatch requests the per-workgroup scan
  // would cost more than it saves, and the padded grid is used as it is.
  int b, s, tile;
  const int max_chunks = a.max_chunks;
  const int chunk = a.device_lengths ? __builtin_amdgcn_readfirstlane(device_chunk(a.cu_prefix, a.batch, max_chunks))
                                     : a.chunk;
  // A single request's bounds are the call's totals (unless the lengths are
  // to be read on the device): nothing is loaded before the first tile's
  // slot indices.
  const bool one = a.batch == 1 && !a.device_lengths;
  const int one_L = a.total_prefix, one_N = a.total_tree;
  auto len_p = [&](int i) -> int { return one ? one_L : a.cu_prefix[i + 1] - a.cu_prefix[i]; };
  auto len_t = [&](int i) -> int { return one ? one_N : a.cu_tree[i + 1] - a.cu_tree[i]; };
  auto nch_of = [&](int L) { return max(1, min((L + chunk - 1) / chunk, max_chunks)); };
  if (a.batch <= kCompactBatch) {
    auto items_of = [&](int i) {
      const int L_i = len_p(i);
      const int rt = min((len_t(i) * a.num_heads + kRowTile - 1) / kRowTile, a.row_tiles);
      return __builtin_amdgcn_readfirstlane(nch_of(L_i) * max(rt, 0));
    };
    int total = 0;
    for (int i = 0; i < a.batch; ++i) total += items_of(i);
    const int per_xcd = (total + 7) >> 3;
    const int j = blockIdx.x >> 3;
    int r = (blockIdx.x & 7) * per_xcd + j;
    if (j >= per_xcd || r >= total) return;
    b = 0;
    for (;;) {
      const int n = items_of(b);
      if (r < n) break;
      r -= n;
      ++b;
    }
    const int rt_b = min((len_t(b) * a.num_heads + kRowTile - 1) / kRowTile, a.row_tiles);
    s = r / rt_b;
    tile = r - s * rt_b;
  } else {
    const int per_xcd = a.grid_items >> 3;
    const int k = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    const int tiles_chunks = a.row_tiles * max_chunks;
    if (k >= a.batch * tiles_chunks) return;
    b = k / tiles_chunks;
    const int rem = k - b * tiles_chunks;
    s = rem / a.row_tiles;
    tile = rem - s * a.row_tiles;
  }
  const int p0 = one ? 0 : a.cu_prefix[b];
  const int L = len_p(b);
  const int nchunks = nch_of(L);
  if (s >= nchunks) return;
  const int kbeg = s * chunk;
  const int kend = min(kbeg + chunk, L);
  const int t0 = one ? 0 : a.cu_tree[b];
  const int n_b = len_t(b);
  const int rows_b = n_b * a.num_heads;
  if (tile * kRowTile >= rows_b) return;
  const int n_tree = min(n_b, kMaxTree);
  const int ntp = kend > kbeg ? (kend - kbeg + kKT - 1) / kKT : 0;
  const int ntt = s == nchunks - 1 ? (n_tree + kKT - 1) / kKT : 0;
  const int ntiles = ntp + ntt;
  const int nfull = (kend - kbeg) / kKT;           // prefix tiles with all 32 keys

  // slot index of key 8c + (lane >> 3) of tile t, for PV wave c
  auto slot_ptr = [&](int t, int c) -> const int* {
    t = min(t, ntiles - 1);
    const bool tree = t >= ntp;
    const int* list = tree ? a.tree_slot + t0 : a.prefix_slot + p0;
    const int base = tree ? (t - ntp) * kKT : kbeg + t * kKT;
    const int last = tree ? n_tree - 1 : kend - 1;
    return list + min(base + 8 * c + (lane >> 3), last);
  };
  // The PV waves read the slot indices of tiles 0..3 before the tree masks
  // are built, so their round trip overlaps that of the parent array.
  uint32_t slot_first[4] = {0u, 0u, 0u, 0u};
  if (!is_qk) {
#pragma unroll
    for (int t = 0; t < 4; ++t) slot_first[t] = (uint32_t)*slot_ptr(t, w - 4);
  }

  // A barrier with no explicit wait: every wave reaches it with its loads
  // issued, so the QK waves' query loads queue behind the slot indices
  // instead of ahead of them (the slots start the dependent slot -> row round
  // trips).  The compiler forms the PV waves' row addresses from the slot
  // values before it, so in practice they reach it once the slots have
  // returned (a cache hit: the index arrays are the same every step).
  __builtin_amdgcn_s_barrier();
  if (ntt > 0) {
    for (int i = threadIdx.x; i < n_tree; i += blockDim.x) sh.par[i] = a.parent[t0 + i];
    __syncthreads();
    if (threadIdx.x < kRowTile) {
      const int r = tile * kRowTile + (int)threadIdx.x;
      int j = r < rows_b ? min(r / a.num_heads, n_tree - 1) : 0;
      uint32_t m[4] = {0u, 0u, 0u, 0u};
      for (int step = 0; step < kMaxTree && j >= 0; ++step) {
        m[j >> 5] |= 1u << (j & 31);
        const int p = sh.par[j];
        j = (p < j) ? p : -1;
      }
      for (int i = 0; i < 4; ++i) sh.vis[threadIdx.x][i] = m[i];
    }
  }

  // The two roles run separate code (separate register sets) in lockstep:
  // both execute the same sequence of barriers.
  //   QK wave w (0..3): pair pr = w >> 1 (rows 32pr..32pr+31), key half
  //     hf = w & 1 (keys 16hf..16hf+15 of each tile).
  //   PV wave c = w - 4 (0..3): output columns [128c, 128c+128), all 64 rows.
  const size_t pidx = ((size_t)b * a.row_tiles + tile) * a.max_chunks + s;
  // more than 16 live rows: the QK waves stage their query rows in LDS (one
  // barrier more in both roles)
  const bool stage_q = __builtin_amdgcn_readfirstlane(rows_b - tile * kRowTile > 16 ? 1 : 0) != 0;
  if (is_qk) {
    const int pr = w >> 1, hf = w & 1, q4 = lane >> 4, l16 = lane & 15;
    // 16-row halves of this pair that hold live query rows (0, 1 or 2): the
    // MFMAs (and, with none live, the K reads) of dead halves are skipped;
    // their scores stay 0, so their P is finite and their rows are dropped
    const int live_pr = rows_b - tile * kRowTile - 32 * pr;
    const int nb_live = __builtin_amdgcn_readfirstlane(live_pr <= 0 ? 0 : live_pr <= 16 ? 1 : 2);
    // Q of the live 16-row halves (a dead half is never multiplied, so it
    // is not loaded: on a 16-row tile that is three quarters of the loads).
    // A tile with more than 16 live rows stages them in LDS first (ring
    // slots 2 and 3, which the loop's first gathers refill only after the
    // prologue barrier), as contiguous kilobytes of q by LDS-DMA, the two
    // waves of a pair taking half of its rows each; after one more barrier
    // each wave reads its fragments from there.  Each row is copied once
    // for both waves, in whole kilobytes: fragment-shaped global loads of
    // the same bytes (16 rows x 64 B per instruction) took twice as long,
    // and loaded every row twice.  A tile of at most 16 rows (one
    // half in one pair) loads its fragments straight from q: there the tile
    // gathers decide when the loop can start.
    bf16x8 qf[kQSteps][2];
    if (stage_q) {
      uint8_t* const qs = pr == 0 ? tile2 : tile3;
      const int live_rows = min(max(live_pr, 0), 32);
      const uint8_t* qpair =
          (const uint8_t*)(a.q + ((size_t)t0 * a.num_heads + tile * kRowTile + 32 * pr) * kDqk);
      const uint32_t m = lds_addr(qs);
      const int nk = __builtin_amdgcn_readfirstlane((live_rows * kDqk * 2 + 1023) >> 10);
      for (int j = 18 * hf; j < min(18 * hf + 18, nk); ++j) {
        const int g = 64 * j + lane;                 // 16-byte slot of the pair's rows
        const int r = g / kChunks16, sl = g - r * kChunks16;
        const int rr = r < live_rows ? r : 0;        // dead rows: any live bytes (zeroed below)
        dma_1k(qpair + (size_t)rr * (kDqk * 2) + ((sl ^ qswz(r)) << 4),
               __builtin_amdgcn_readfirstlane(m + 1024 * j));
      }
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int r = 16 * nb + l16;
        const bool ok = r < live_rows;
        const uint8_t* qrow = qs + r * (kDqk * 2);
        if (nb < nb_live) {
#pragma unroll
          for (int st = 0; st < kQSteps; ++st) {
            const bf16x8 v = *(const bf16x8*)(qrow + (((4 * st + q4) ^ qswz(r)) << 4));
            qf[st][nb] = ok ? v : bf16x8{};
          }
        } else {
#pragma unroll
          for (int st = 0; st < kQSteps; ++st) qf[st][nb] = bf16x8{};
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = tile * kRowTile + 32 * pr + 16 * nb + l16;
        const bool ok = row < rows_b;
        const uint16_t* qrow = a.q + ((size_t)t0 * a.num_heads + (ok ? row : 0)) * kDqk;
        if (nb < nb_live) {
#pragma unroll
          for (int st = 0; st < kQSteps; ++st) {
            const bf16x8 v = *(const bf16x8*)(qrow + (4 * st + q4) * 8);
            qf[st][nb] = ok ? v : bf16x8{};
          }
        } else {
#pragma unroll
          for (int st = 0; st < kQSteps; ++st) qf[st][nb] = bf16x8{};
        }
      }
    }
    // K fragment of step st: key 16hf + l16 = unit 2hf + (l16 >> 3), key
    // l16 & 7 of it; pieces 4st + q4 = group st >> 1, piece 4(st & 1) + q4
    const int k8 = l16 & 7;
    const int qk_base = (2 * hf + (l16 >> 3)) * kUnit + k8 * 128 + ((q4 ^ swz(k8)) << 4);
    float m_ref[2] = {-INFINITY, -INFINITY};   // rows 16nb + l16 of the pair
    float lsum[2] = {0.f, 0.f};
    bool have_ref = false;
    int restart_tile = 0;
    int restarts = 0;
    // max of row 16nb + l16 of the pair over tile slot k: its four lanes in
    // this wave and in the partner wave
    auto pair_row_max = [&](int k, int nb) {
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float2 u = sh.mtl[k][w][16 * q + l16], v = sh.mtl[k][w ^ 1][16 * q + l16];
        m = fmaxf(m, fmaxf(nb ? u.y : u.x, nb ? v.y : v.x));
      }
      return m;
    };
    for (;;) {                                 // again after a restart
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();                         // prologue: tiles 0, 1 staged
      bool restart = false;
      // Iteration it scores tile it and turns the scores of tile it-1 into
      // P; the PV waves consume P(it-2).  The softmax runs while this
      // tile's first K fragments are in flight.
      f32x4 sprev[2] = {f32x4{}, f32x4{}};   // masked scores of tile it-1
      int mi = 0;                            // it mod 3
      float mprev[2] = {0.f, 0.f};           // their row max (log2 units), this wave's keys
      for (int it = 0; it <= ntiles + 1; ++it) {
        typedef __attribute__((address_space(3))) const bf16x8 lds_frag;
        const uint32_t slot = lds_addr(ring(it));
        const lds_frag* kp[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) kp[j] = (const lds_frag*)(uintptr_t)(slot + (uint32_t)(qk_base ^ (64 * j)));
        auto kfrag = [&](int st) { return kp[st & 1][(kGroup / 16) * (st >> 1)]; };
        // restart vote on tile it-2 (its softmax ran in the iteration before),
        // read ahead of the K fragments so that its wait does not cover them
        f32x4 vote = f32x4{};
        if (it >= 2) vote = *(const f32x4*)sh.want[it & 1];
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 kf[kPreQK];
        if (it < ntiles && nb_live > 0) {
#pragma unroll
          for (int i = 0; i < kPreQK; ++i) kf[i] = kfrag(i);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (it >= 1 && it <= ntiles) {
          const int t = it - 1;
          if (t == 0 && !have_ref) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) m_ref[nb] = pair_row_max(0, nb) + kMargin;
          }
          // P in bf16, stored in the PV B-operand layout: block (ks = hf,
          // rb = pr), lane L = j + 32*(q4 >> 1) holds keys 8*(q4 >> 1) .. +7 of
          // row j; this lane's 4 keys are bytes 8*(q4 & 1) .. +7 of it
          uint8_t* pbl = sh.pbuf[t & 1][2 * hf + pr];
          bool want = false;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            float ps[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ps[r] = __builtin_amdgcn_exp2f(fmaf(sprev[nb][r], a.scale_log2, -m_ref[nb]));
            lsum[nb] += (ps[0] + ps[1]) + (ps[2] + ps[3]);
            typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
            bf16x4 pk;
#pragma unroll
            for (int r = 0; r < 4; ++r) pk[r] = (__bf16)ps[r];
            const int j = 16 * nb + l16;
            *(bf16x4*)(pbl + (j + 32 * (q4 >> 1)) * 16 + 8 * (q4 & 1)) = pk;
            want |= mprev[nb] > m_ref[nb] + kSlack;
          }
          // every lane stores the wave's vote (same value, same address)
          sh.want[t & 1][w] = __any(want) ? 1.f : 0.f;
        }
        if (it < ntiles) {
          f32x4 sacc[2] = {f32x4{}, f32x4{}};
          if (nb_live == 2) {
#pragma unroll
            for (int st = 0; st < kQSteps; ++st) {
              const bf16x8 cur = kf[st % kPreQK];
              if (st + kPreQK < kQSteps) kf[st % kPreQK] = kfrag(st + kPreQK);
              sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qf[st][0], sacc[0], 0, 0, 0);
              sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qf[st][1], sacc[1], 0, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else if (nb_live == 1) {
#pragma unroll
            for (int st = 0; st < kQSteps; ++st) {
              const bf16x8 cur = kf[st % kPreQK];
              if (st + kPreQK < kQSteps) kf[st % kPreQK] = kfrag(st + kPreQK);
              sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qf[st][0], sacc[0], 0, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // lane holds keys 16hf + 4q4 + r (r = 0..3) of rows 32pr + 16nb + l16
          // masks only on the last prefix tile (ragged) and the tree tiles
          if (it >= nfull) {
            const bool tree = it >= ntp;
            const int nvalid = tree ? kKT : min(kKT, kend - kbeg - it * kKT);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              if (nvalid < kKT) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (16 * hf + 4 * q4 + r >= nvalid) sacc[nb][r] = -INFINITY;
              }
              if (tree) {
                const uint32_t vm = sh.vis[32 * pr + 16 * nb + l16][it - ntp];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (((vm >> (16 * hf + 4 * q4 + r)) & 1u) == 0) sacc[nb][r] = -INFINITY;
              }
            }
          }
          // this lane's max over its 4 keys of each row (log2 units): a row
          // breaks the reference iff one of its lanes does, so the restart
          // test needs no cross-lane reduction; the row max itself is
          // reduced only on the rare paths (first tile, restart)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            mprev[nb] = vmax(vmax(sacc[nb][0], sacc[nb][1]), vmax(sacc[nb][2], sacc[nb][3])) * a.scale_log2;
          sh.mtl[mi][w][lane] = make_float2(mprev[0], mprev[1]);
          sprev[0] = sacc[0];
          sprev[1] = sacc[1];
        }
        // restart vote on tile it-2, taken at the end of the iteration so
        // that its LDS wait lands where the barrier waits anyway
        if ((vote[0] + vote[1]) + (vote[2] + vote[3]) != 0.f) {
          restart = true;
          restart_tile = it - 2;
          break;
        }
        mi = mi == 2 ? 0 : mi + 1;
        lds_barrier();
      }
      if (!restart) break;
      ++restarts;
      // restart with each row's reference raised to its max over the
      // offending tile + kMargin
      const int bad = restart_tile % 3;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        m_ref[nb] = fmaxf(m_ref[nb], pair_row_max(bad, nb) + kMargin);
        lsum[nb] = 0.f;
      }
      have_ref = true;
      __syncthreads();
    }
    if (a.debug_record && restarts > 0 && w == 0 && lane == 0)
      atomicAdd(const_cast<int32_t*>(a.debug_record) + 3, restarts);
    // row sums: the four lanes of the row, then the partner wave
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) lsum[nb] = sum4(lsum[nb]);
    sh.mtl[0][w][lane].x = q4 == 0 ? lsum[0] : lsum[1];
    lds_barrier();
    if (hf == 0 && q4 < 2) {
      const int j = 32 * pr + lane;
      const float l = sh.mtl[0][w][lane].x + sh.mtl[0][w ^ 1][lane].x;
      sh.rowl[j] = l;
      if (tile * kRowTile + j < rows_b) {
        const float v = m_ref[q4] * kLn2 + logf(l);
        if (a.out) a.lse[(size_t)t0 * a.num_heads + tile * kRowTile + j] = v;   // the request's only chunk
        else a.part_lse[pidx * kRowTile + j] = v;
      }
    }
    lds_barrier();
    return;
  }

  // ---------------- PV waves ----------------
  const int c = w - 4;
  // rows 32..63 of the tile: with none live their MFMAs are skipped (a
  // uniform branch around each; the LDS reads, and so the hand-counted
  // waits, stay as they are)
  const bool rb1_live = __builtin_amdgcn_readfirstlane(rows_b - tile * kRowTile > 32 ? 1 : 0) != 0;
  f32x16 o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = f32x16{};
  // transposed V reads: lane (block bb = lane/16, e = (lane/4)%4, s2 = lane%4)
  // reads columns 128c + 32cb + 16(bb & 1) + 4s2 .. +3 of key
  // 16ks + 8(bb >> 1) + e + 4hi: unit 2ks + (bb >> 1), key e + 4hi of it,
  // piece 16c + 4cb + 2(bb & 1) + (s2 >> 1) = group 2c + (cb >> 1), piece
  // 4(cb & 1) + 2(bb & 1) + (s2 >> 1) of the group, half s2 & 1 of the piece
  int pvb[2];
  {
    const int bb = lane >> 4, e = (lane >> 2) & 3, s2 = lane & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int kk = e + 4 * hi;
      pvb[hi] = (bb >> 1) * kUnit + 2 * c * kGroup + kk * 128 + (((2 * (bb & 1) + (s2 >> 1)) ^ swz(kk)) << 4) +
                8 * (s2 & 1);
    }
  }
  // this lane's piece offset inside a row (see gather_tile)
  const uint8_t* pool_lane = (const uint8_t*)a.pool + (((lane & 7) ^ swz(lane >> 3)) << 4);
  // slots of tile t; valid after the next vmcnt wait
  auto load_slot = [&](int t) -> uint32_t { return load_u32_async(slot_ptr(t, c)); };
  // tiles 0 and 1 are in flight while the QK waves stage their query rows
  // (the barrier after which those rows have landed in ring slots 2 and 3);
  // a restart gathers them again
  gather_tile(pool_lane, slot_first[0], tile0, c);
  if (ntiles > 1) gather_tile(pool_lane, slot_first[1], tile1, c);
  if (stage_q) asm volatile("s_barrier" ::: "memory");
  for (bool again = false;; again = true) {
    // Slot ring: svd holds the slots of tile it+2 (gathered in iteration it),
    // svn those of tile it+3.  Each iteration loads the next slots before its
    // gathers, so the in-order vector-memory counter never makes a slot load
    // wait for a gather.
    uint32_t svd = slot_first[2], svn = slot_first[3];
    if (again) {
      gather_tile(pool_lane, slot_first[0], tile0, c);
      if (ntiles > 1) gather_tile(pool_lane, slot_first[1], tile1, c);
    }
    // tile 0 must have landed; tile 1's nine gathers may stay in flight
    // (iteration 0's closing wait covers them)
    if (ntiles > 1) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // V^T fragment f = 4ks + cb: two transposed reads at
    // slot + vad[cb & 1][hi] + (2 units) ks + (1 group) (cb >> 1)
    uint32_t vad[2][2];
#pragma unroll
    for (int cp = 0; cp < 2; ++cp)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) vad[cp][hi] = (uint32_t)(pvb[hi] ^ (64 * cp));
    auto vread = [&](uint32_t slot, int f) {
      const int ks = f >> 2, cb = f & 3;
      const int off = ks * 2 * kUnit + (cb >> 1) * kGroup;
      const i16x4 lo = ds_tr(slot + vad[cb & 1][0], off);
      const i16x4 hi = ds_tr(slot + vad[cb & 1][1], off);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    const uint32_t pb_addr[2] = {lds_addr(sh.pbuf[0][0]) + 16 * lane, lds_addr(sh.pbuf[1][0]) + 16 * lane};
    const uint32_t want_addr[2] = {lds_addr(sh.want[0]), lds_addr(sh.want[1])};
    // V^T fragments: iteration it multiplies V(it-2) by P(it-2) and reads
    // V(it-1) into each fragment register right after its last use
    bf16x8 vf[8];
    bool restart = false;
    for (int it = 0; it <= ntiles + 1; ++it) {
      const bool do_dma = it + 2 < ntiles;
      uint8_t* dbuf = ring(it + 2);
      const uint32_t nslot = lds_addr(ring(max(it - 1, 0)));
      uint32_t svf = load_slot(it + 4);           // issued before this iteration's gathers
      f32x4 vote = f32x4{};
      if (it >= 2) {
        // LDS operations in issue order: vote, P0..P3, then two per fragment
        vote = __builtin_bit_cast(f32x4, ds_b128(want_addr[it & 1], 0));
        bf16x8 pop[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pop[i] = ds_b128(pb_addr[it & 1], i * 1024);
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          const int ks = f >> 2, cb = f & 3;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const int j = 2 * ks + rb;
            if (cb == 0) wait_lgkm((3 - j) + 2 * f, pop[j]);
            if (rb == 0 || rb1_live)
              o[cb + 4 * rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[f], pop[j], o[cb + 4 * rb], 0, 0, 0);
            if (rb == 1) vf[f] = vread(nslot, f);  // V(it-1); at it = ntiles+1 a harmless re-read
            __builtin_amdgcn_sched_barrier(0);
          }
          // the gather of tile it+2, issued once the first four MFMAs are
          // under way: issued before them, its address arithmetic kept the
          // matrix core idle at the top of the iteration; issued later, the
          // rows arrive late
          if (f == 1 && do_dma) {
            gather_tile(pool_lane, svd, dbuf, c);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
        if (it == 1) {
#pragma unroll
          for (int f = 0; f < 8; ++f) vf[f] = vread(nslot, f);
        }
        if (do_dma) {
          gather_tile(pool_lane, svd, dbuf, c);
        }
      }
      // the gather of tile it+1 (issued one iteration ago) and the slot load
      // above must have landed; this iteration's nine gathers may stay in
      // flight (vector memory completes in order)
      if (do_dma) asm volatile("s_waitcnt vmcnt(9)" : "+v"(svf) :: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" : "+v"(svf) :: "memory");
      svd = svn;
      svn = svf;
      // V(it-1) reads landed (and named, for their next use) before the barrier
      // after which their slot may be refilled
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(vote), "+v"(vf[0]), "+v"(vf[1]), "+v"(vf[2]), "+v"(vf[3]), "+v"(vf[4]), "+v"(vf[5]),
                     "+v"(vf[6]), "+v"(vf[7])
                   :
                   : "memory");
      if ((vote[0] + vote[1]) + (vote[2] + vote[3]) != 0.f) {   // restart vote on tile it-2
        restart = true;
        break;
      }
      asm volatile("s_barrier" ::: "memory");
    }
    if (!restart) break;
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = f32x16{};
    __syncthreads();
  }
  lds_barrier();                                  // QK waves publish row sums
  lds_barrier();
  float* po = a.part_o + pidx * (kD4 * kRowTile * 4);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int rit = 32 * rb + (lane & 31);
    if (tile * kRowTile + rit >= rows_b) continue;
    const float inv = __builtin_amdgcn_rcpf(sh.rowl[rit]);   // <= 1 ulp
    // the request's only chunk: its normalised partial is the output (a
    // merge of one partial multiplies it by exactly 1), rounded to bf16
    uint16_t* orow = a.out ? a.out + ((size_t)t0 * a.num_heads + tile * kRowTile + rit) * kDv : nullptr;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d4 = (4 * c + cb) * 8 + 2 * rq + (lane >> 5);
        const f32x16& acc = o[cb + 4 * rb];
        const float4 v = make_float4(acc[4 * rq] * inv, acc[4 * rq + 1] * inv, acc[4 * rq + 2] * inv,
                                     acc[4 * rq + 3] * inv);
        if (orow) {
          uint2 pk;
          pk.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.x) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.y) << 16);
          pk.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.z) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.w) << 16);
          *(uint2*)(orow + d4 * 4) = pk;
        } else {
          *(float4*)(po + ((size_t)d4 * kRowTile + rit) * 4) = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_prefix_splitkv(const PrefixArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(prefix_splitkv_kernel, dim3(a.grid_items), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace vamla
