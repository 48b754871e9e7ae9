"""Seeded synthetic inputs for DDTree verify attention over an MLA latent pool.

This module draws every input both the HIP path and the CPU oracle consume:
tree shapes (parent arrays), slot lists into a page_size=1 pool, the pool's
latent rows and the queries.  It holds none of the attention arithmetic; the
only numeric step here is rounding the drawn fp32 values to bf16 bit patterns
(round to nearest, ties to even), which both sides then read as identical bits.

Workload shapes follow the pages:
  * "Mapping the Kernel Frontier", section "The Context: A Hard-Earned
    Diagnosis": batch 1 with 9 verify queries over a long context.
  * "The Architecture Detective: ...", section "The Message in Full": the tree
    has at most 65 nodes; every node attends the whole prefix; the pool holds one
    576-wide latent row per token (num_heads_k = 1, head_dim = 576).
  * Same page, "Defragmentation: Separating Signal from Noise", and "The Anatomy
    of a Kernel Investigation", section "The Bash Command": the allocator hands
    out the head of a free list, appends freed slots at its tail, and slot 0 is
    reserved padding.  `churned_allocator` replays that policy to produce a
    realistically scrambled pool.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

D_QK = 576          # 512 latent + 64 rope
D_V = 512           # V is the first 512 columns of the same row
SOFTMAX_SCALE = 1.0 / math.sqrt(192.0)
BF16_NAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# bf16 bit patterns
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction (normal draws), so no NaN handling.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, std: float = 0.1) -> np.ndarray:
    """N(0, 1) * std drawn in fp32 with PCG64, rounded to bf16 bits."""
    vals = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(vals)


# --------------------------------------------------------------------------
# trees (request-local parent arrays, parent[0] = -1, 0 <= parent[i] < i)
# --------------------------------------------------------------------------

def random_tree(n: int, rng: np.random.Generator) -> np.ndarray:
    """parent[i] ~ U[0, i) for i >= 1."""
    parent = np.full(n, -1, dtype=np.int32)
    for i in range(1, n):
        parent[i] = int(rng.integers(0, i))
    return parent


def chain_plus_branch(chain: int = 8, branch_parent: int = 0) -> np.ndarray:
    """A chain of `chain` nodes (root included: node i's parent is i-1), then
    one extra node hanging off `branch_parent` (for the default, a sibling of
    node 1: the drafter's second choice for the first token)."""
    parent = np.arange(-1, chain - 1, dtype=np.int32)
    return np.concatenate([parent, np.array([branch_parent], dtype=np.int32)])


def bounded_tree(n: int, rng: np.random.Generator, max_depth: int = 8,
                 max_children: int = 4) -> np.ndarray:
    """Nodes 1..max_depth form a chain (so the depth bound is reached); every
    later node picks a parent uniformly among earlier nodes whose depth is
    below max_depth and who have fewer than max_children children."""
    parent = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int32)
    children = np.zeros(n, dtype=np.int32)
    for i in range(1, n):
        if i <= max_depth:
            p = i - 1
        else:
            cand = [v for v in range(i) if depth[v] < max_depth and children[v] < max_children]
            if not cand:
                raise ValueError("tree bounds leave no legal parent")
            p = cand[int(rng.integers(0, len(cand)))]
        parent[i] = p
        depth[i] = depth[p] + 1
        children[p] += 1
    return parent


def tree_depths(parent: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parent), dtype=np.int32)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


def all_parent_arrays(n: int):
    """Every topologically ordered parent array with n nodes (prod_{i<n} i of them)."""
    if n <= 0:
        return
    def rec(i, cur):
        if i == n:
            yield np.array(cur, dtype=np.int32)
            return
        for p in range(i):
            yield from rec(i + 1, cur + [p])
    yield from rec(1, [-1])


# --------------------------------------------------------------------------
# slot allocation
# --------------------------------------------------------------------------

class FreeListAllocator:
    """page_size=1 free list: alloc(n) takes the first n free slots, free()
    appends slots to the end.  Slot 0 is never handed out.  Backed by a ring
    buffer so 2M-slot pools stay cheap.

    sorted=True keeps the free list in slot order instead: alloc(n) takes the
    n lowest free slots (a bitmap of free slots), so freed holes are refilled
    first and long runs stay free at the top of the pool."""

    def __init__(self, pool_slots: int, sorted: bool = False):
        self.cap = pool_slots
        self.sorted = sorted
        self.size = pool_slots - 1
        if sorted:
            self.free_mask = np.ones(pool_slots, dtype=bool)
            self.free_mask[0] = False
        else:
            self.ring = np.zeros(pool_slots, dtype=np.int64)
            self.ring[: pool_slots - 1] = np.arange(1, pool_slots, dtype=np.int64)
            self.head = 0

    def alloc(self, n: int) -> np.ndarray:
        if n > self.size:
            raise MemoryError("pool exhausted")
        if self.sorted:
            out = np.flatnonzero(self.free_mask)[:n].astype(np.int64)
            self.free_mask[out] = False
        else:
            idx = (self.head + np.arange(n)) % self.cap
            out = self.ring[idx].copy()
            self.head = (self.head + n) % self.cap
        self.size -= n
        return out

    def free(self, slots: np.ndarray) -> None:
        n = len(slots)
        if self.sorted:
            self.free_mask[slots] = True
        else:
            tail = (self.head + self.size) % self.cap
            idx = (tail + np.arange(n)) % self.cap
            self.ring[idx] = slots
        self.size += n


def churned_allocator(pool_slots: int, reserve: int, rng: np.random.Generator,
                      n_requests: int = 10_000, lo: int = 64, hi: int = 16384,
                      sorted: bool = False) -> FreeListAllocator:
    """Replay `n_requests` allocations with sizes ~ logU[lo, hi]; before each
    alloc, free random live requests until the free list holds size + reserve;
    after each alloc, free one random live request with probability 1/2.
    sorted selects the sorted free list (lowest free slots first)."""
    a = FreeListAllocator(pool_slots, sorted=sorted)
    live: List[np.ndarray] = []
    llo, lhi = math.log(lo), math.log(hi)
    for _ in range(n_requests):
        size = int(round(math.exp(rng.uniform(llo, lhi))))
        while a.size < size + reserve and live:
            j = int(rng.integers(0, len(live)))
            a.free(live.pop(j))
        live.append(a.alloc(size))
        if live and rng.random() < 0.5:
            j = int(rng.integers(0, len(live)))
            a.free(live.pop(j))
    return a


# --------------------------------------------------------------------------
# full verify inputs
# --------------------------------------------------------------------------

@dataclasses.dataclass
class VerifyInputs:
    """Host copies of one verify step's inputs (bf16 as uint16 bits)."""
    q: np.ndarray                 # [T, H, 576] uint16
    pool: np.ndarray              # [P, 576] uint16
    prefix_slot_idx: np.ndarray   # [sum L_b] int32
    tree_slot_idx: np.ndarray     # [T] int32
    parent: np.ndarray            # [T] int32, request-local
    cu_prefix: np.ndarray         # [B+1] int32
    cu_tree: np.ndarray           # [B+1] int32
    num_heads: int
    scale: float = SOFTMAX_SCALE
    seed_info: str = ""

    @property
    def batch(self) -> int:
        return len(self.cu_prefix) - 1

    @property
    def total_tree(self) -> int:
        return int(self.cu_tree[-1])

    @property
    def total_prefix(self) -> int:
        return int(self.cu_prefix[-1])

    def prefix_len(self, b: int) -> int:
        return int(self.cu_prefix[b + 1] - self.cu_prefix[b])

    def tree_len(self, b: int) -> int:
        return int(self.cu_tree[b + 1] - self.cu_tree[b])


def make_inputs(prefix_lens: Sequence[int], parents: Sequence[np.ndarray], num_heads: int,
                pool_slots: int, slot_mode: str, seed: int, std_q: float = 0.1,
                std_kv: float = 0.1, poison_unused: bool = True,
                churn_requests: int = 10_000) -> VerifyInputs:
    """Build one batch.  slot_mode in {"contiguous", "scrambled", "churned",
    "churned_sorted"} (the last two replay the free-list or the sorted-free-list
    allocator).

    Streams spawned from SeedSequence(seed): [tree-independent] slots, pool, q.
    Logical rows (prefix then tree, per request) get their values in logical
    order, so two slot modes with the same seed hold identical logical data.
    """
    ss = np.random.SeedSequence(seed)
    s_slots, s_pool, s_q = [np.random.default_rng(s) for s in ss.spawn(3)]
    B = len(prefix_lens)
    assert len(parents) == B
    Ls = [int(x) for x in prefix_lens]
    Ns = [len(p) for p in parents]
    need = sum(Ls) + sum(Ns)
    if need > pool_slots - 1:
        raise ValueError("pool too small for the requested rows")

    if slot_mode == "contiguous":
        logical_slots = np.arange(1, need + 1, dtype=np.int64)
    elif slot_mode == "scrambled":
        logical_slots = s_slots.permutation(np.arange(1, pool_slots, dtype=np.int64))[:need]
    elif slot_mode in ("churned", "churned_sorted"):
        alloc = churned_allocator(pool_slots, need, s_slots, n_requests=churn_requests,
                                  sorted=slot_mode == "churned_sorted")
        parts = []
        for b in range(B):
            parts.append(alloc.alloc(Ls[b]))
        for b in range(B):
            parts.append(alloc.alloc(Ns[b]))
        # reorder to (prefix_0, ..., prefix_{B-1}, tree_0, ...) -> keep as is
        logical_slots = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    else:
        raise ValueError(slot_mode)

    total_L = sum(Ls)
    prefix_slots = logical_slots[:total_L].astype(np.int32)
    tree_slots = logical_slots[total_L:].astype(np.int32)

    pool = np.empty((pool_slots, D_QK), dtype=np.uint16)
    pool[:] = BF16_NAN if poison_unused else np.uint16(0)
    # values drawn in logical order: prefix rows of all requests, then tree rows
    vals = normal_bf16(s_pool, (need, D_QK), std_kv)
    pool[logical_slots] = vals

    T = sum(Ns)
    q = normal_bf16(s_q, (T, num_heads, D_QK), std_q)
    cu_prefix = np.zeros(B + 1, dtype=np.int32)
    cu_prefix[1:] = np.cumsum(Ls)
    cu_tree = np.zeros(B + 1, dtype=np.int32)
    cu_tree[1:] = np.cumsum(Ns)
    parent = np.concatenate([np.asarray(p, dtype=np.int32) for p in parents]) if B else np.zeros(0, np.int32)
    return VerifyInputs(q=q, pool=pool, prefix_slot_idx=prefix_slots, tree_slot_idx=tree_slots,
                        parent=parent, cu_prefix=cu_prefix, cu_tree=cu_tree, num_heads=num_heads,
                        seed_info=f"seed={seed} slots={slot_mode}")


# --------------------------------------------------------------------------
# the five workload configurations
# --------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny: B=1 H=16 L=1024 N=9 random tree, 4096-slot scrambled pool",
    2: "B=1 H=16 L=8192 N=9 chain-of-8-plus-branch, 32768-slot pool (contiguous|scrambled)",
    3: "B=1 H=16 L=65536 N=65 depth-8 branching<=4 tree, 131072-slot scrambled pool",
    4: "B=1 H=128 L=131072 N=65 depth-8 tree, 2^20-slot churned pool",
    5: "B=8 H=16 L~logU[4096,185000] N=33 depth<=8 trees, shared 2^21-slot churned pool",
    # small-rows regime (fewer query rows than the ~315 flop/byte ridge needs:
    # the step is bound by reading KV from HBM)
    6: "decode: B=1 H=16 L=131072 N=1 (root only), 262144-slot scrambled pool",
    7: "B=1 H=16 L=185000 N=9 chain-of-8-plus-branch, 262144-slot scrambled pool",
}


def config_inputs(k: int, slot_mode: Optional[str] = None, std_q: float = 0.1,
                  poison_unused: bool = True, prefix: Optional[int] = None) -> VerifyInputs:
    """Inputs of workload configuration k (1..7); seeds derive from 1000*k.
    prefix replaces the prefix length of a single-request workload (the tree,
    heads, pool size and seeds stay those of workload k)."""
    seed = 1000 * k
    tree_rng = np.random.default_rng(np.random.SeedSequence(seed + 7))
    if prefix is not None and (k == 5 or prefix < 0):
        raise ValueError("prefix applies to the single-request workloads (1-4, 6, 7), as a length >= 0")
    L = (lambda default: default if prefix is None else prefix)
    if k == 1:
        return make_inputs([L(1024)], [random_tree(9, tree_rng)], 16, max(4096, L(0) + 4096),
                           slot_mode or "scrambled", seed, std_q=std_q, poison_unused=poison_unused)
    if k == 2:
        return make_inputs([L(8192)], [chain_plus_branch()], 16, max(32768, L(0) + 4096),
                           slot_mode or "scrambled", seed, std_q=std_q, poison_unused=poison_unused)
    if k == 3:
        return make_inputs([L(65536)], [bounded_tree(65, tree_rng)], 16, max(131072, L(0) + 4096),
                           slot_mode or "scrambled", seed, std_q=std_q, poison_unused=poison_unused)
    if k == 4:
        return make_inputs([L(131072)], [bounded_tree(65, tree_rng)], 128, max(1 << 20, L(0) + 4096),
                           slot_mode or "churned", seed, std_q=std_q, poison_unused=poison_unused)
    if k == 5:
        lens = [int(round(math.exp(tree_rng.uniform(math.log(4096), math.log(185000)))))
                for _ in range(8)]
        trees = [bounded_tree(33, tree_rng) for _ in range(8)]
        return make_inputs(lens, trees, 16, 1 << 21, slot_mode or "churned", seed,
                           std_q=std_q, poison_unused=poison_unused)
    if k == 6:
        return make_inputs([L(131072)], [np.array([-1], np.int32)], 16, max(1 << 18, L(0) + 4096),
                           slot_mode or "scrambled", seed, std_q=std_q, poison_unused=poison_unused)
    if k == 7:
        return make_inputs([L(185000)], [chain_plus_branch()], 16, max(1 << 18, L(0) + 4096),
                           slot_mode or "scrambled", seed, std_q=std_q, poison_unused=poison_unused)
    raise ValueError(k)
