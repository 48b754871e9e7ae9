"""Host-side slot management of the page_size=1 latent KV pool: allocation,
the Tier-0 compaction policy and the accepted-path commit of a verify step.

The pages describe the pieces this module puts together:
  * "The Architecture Detective: ...", "Defragmentation: Separating Signal
    from Noise": a page_size=1 allocator hands out the head of a free list and
    appends freed slots at its tail, so after churn a request's rows are
    scattered; compaction moves them into a contiguous run.  Its value depends
    on the churn and is secondary to the kernel.
  * "The Anatomy of a Kernel Investigation", "Conclusion": the live service ran
    Tier-0 defragmentation next to the graph-captured verify kernel.
  * "Mapping the Kernel Frontier", "The Context: A Hard-Earned Diagnosis": the
    verify step's accepted tokens join the request's context; their rows were
    written to scattered tree slots.
  * "The Anatomy of a Kernel Investigation", "The Bash Command": slot 0 is
    padding and is never handed out.

Every row move goes through vamla_slot_gather (bit-exact, on the GPU); this
module only decides which slots, keeps the slot tables and never touches row
contents on the host.  The verify kernels read rows by logical position, so
moving a request's rows changes no result bit (a property the tests check).
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from . import binding as vb


class SlotAllocator:
    """Free slots of a pool of `pool_slots` rows (slot 0 reserved).

    policy "fifo": alloc(n) takes the n slots at the head of the free list and
    free() appends at its tail (the allocator the pages describe).
    policy "sorted": the free list is kept in slot order and alloc(n) takes the
    n lowest free slots, so consecutive allocations tend to be contiguous.

    find_run / take_run / alloc_run hand out contiguous runs whatever the
    policy (the compaction targets).  A bitmap of free slots backs the run
    searches; in fifo mode the ring always holds exactly the free slots, in
    free-list order (a run claim removes its slots from it).
    """

    def __init__(self, pool_slots: int, policy: str = "fifo"):
        if policy not in ("fifo", "sorted"):
            raise ValueError(policy)
        if pool_slots < 2:
            raise ValueError("pool needs at least one slot besides the padding slot 0")
        self.pool_slots = int(pool_slots)
        self.policy = policy
        self.is_free = np.zeros(self.pool_slots, dtype=bool)
        self.is_free[1:] = True
        self._ring = np.zeros(self.pool_slots, dtype=np.int64)
        self._ring[: self.pool_slots - 1] = np.arange(1, self.pool_slots)
        self._head = 0
        self.n_free = self.pool_slots - 1

    def _ring_view(self) -> np.ndarray:
        idx = (self._head + np.arange(self.n_free)) % self.pool_slots
        return self._ring[idx]

    def alloc(self, n: int) -> np.ndarray:
        if n < 0 or n > self.n_free:
            raise MemoryError(f"cannot allocate {n} slots ({self.n_free} free)")
        if self.policy == "sorted":
            out = np.flatnonzero(self.is_free)[:n].astype(np.int64)
        else:
            idx = (self._head + np.arange(n)) % self.pool_slots
            out = self._ring[idx].copy()
            self._head = (self._head + n) % self.pool_slots
        self.is_free[out] = False
        self.n_free -= n
        return out

    def free(self, slots: Sequence[int]) -> None:
        s = np.asarray(slots, dtype=np.int64).ravel()
        if s.size == 0:
            return
        if (s <= 0).any() or (s >= self.pool_slots).any():
            raise ValueError("slot out of range (slot 0 is padding)")
        if self.is_free[s].any() or len(np.unique(s)) != s.size:
            raise ValueError("double free")
        if self.policy == "fifo":
            tail = (self._head + self.n_free) % self.pool_slots
            idx = (tail + np.arange(s.size)) % self.pool_slots
            self._ring[idx] = s
        self.is_free[s] = True
        self.n_free += s.size

    def find_run(self, n: int) -> Optional[int]:
        """Start of the lowest run of n free slots, or None."""
        if n <= 0:
            raise ValueError("run length must be positive")
        d = np.diff(np.concatenate([[0], self.is_free.astype(np.int8), [0]]))
        starts = np.flatnonzero(d == 1)
        ends = np.flatnonzero(d == -1)
        ok = np.flatnonzero(ends - starts >= n)
        return int(starts[ok[0]]) if ok.size else None

    def take_run(self, start: int, n: int) -> np.ndarray:
        """Claim slots [start, start+n), which must all be free."""
        s = np.arange(start, start + n, dtype=np.int64)
        if start < 1 or start + n > self.pool_slots or not self.is_free[s].all():
            raise ValueError("run not free")
        if self.policy == "fifo":
            live = self._ring_view()
            live = live[(live < start) | (live >= start + n)]
            self._ring[: live.size] = live
            self._head = 0
        self.is_free[s] = False
        self.n_free -= n
        return s

    def alloc_run(self, n: int) -> Optional[np.ndarray]:
        start = self.find_run(n)
        return None if start is None else self.take_run(start, n)


def count_runs(slots: Sequence[int]) -> int:
    """Contiguous runs of a slot list in logical order (1 = fully contiguous)."""
    s = np.asarray(slots, dtype=np.int64)
    if s.size == 0:
        return 0
    return int(1 + np.count_nonzero(np.diff(s) != 1))


@dataclasses.dataclass
class Request:
    """Slot table of one request: its prefix rows in logical order, and free
    slots reserved right after them for the tokens it will accept."""
    prefix: np.ndarray
    reserve: np.ndarray = dataclasses.field(default_factory=lambda: np.zeros(0, dtype=np.int64))

    @property
    def length(self) -> int:
        return int(len(self.prefix))


def accepted_path(parent: Sequence[int], leaf: int) -> List[int]:
    """Tree nodes from the root to `leaf` (request-local indices), root first."""
    path = []
    j = int(leaf)
    while j >= 0:
        path.append(j)
        j = int(parent[j])
    return path[::-1]


class Tier0Defrag:
    """The Tier-0 policy: keep long-lived requests in contiguous runs when
    that pays.

    compact(req) moves a request's prefix rows into one contiguous run, with
    `headroom` free slots after it reserved for the tokens the request will
    accept, when its rows are split over more than one run and such a run is
    free.  should_compact(req, expected_steps) prices that one-time copy
    against the per-step gain of a contiguous layout: compact when
    expected_steps * step_gain_us >= rows * gather_us_per_row.  Both figures
    are measurements (bench.py --defrag: the step on scattered and on
    contiguous slots, and the gather's rate); with this library's verify
    kernel the per-step gain measured on the 8k-prefix and 128k-prefix decode
    workloads is nil (the kernel reads each 1152-byte row whole, wherever it
    sits), so the default step_gain_us = 0 never compacts.

    commit_accepted(req, ...) appends the accepted path of a verified tree to
    the request: its rows move from their scattered tree slots into the
    request's reserve (or the free slots right after its run, or else a new
    run of their own), and every tree slot of the step is freed.  That move is
    at most 65 rows, so it is done whatever the policy.
    """

    def __init__(self, allocator: SlotAllocator, step_gain_us: float = 0.0, gather_us_per_row: float = 0.39e-3,
                 headroom: int = 64):
        self.alloc = allocator
        self.step_gain_us = float(step_gain_us)
        self.gather_us_per_row = float(gather_us_per_row)
        self.headroom = int(headroom)

    def payback_steps(self, req: Request) -> float:
        """Steps after which compacting req pays back (inf when never)."""
        if self.step_gain_us <= 0:
            return float("inf")
        return req.length * self.gather_us_per_row / self.step_gain_us

    def should_compact(self, req: Request, expected_steps: float) -> bool:
        return count_runs(req.prefix) > 1 and expected_steps >= self.payback_steps(req)

    def release(self, req: Request) -> None:
        """Free the request's rows and reserve (request finished)."""
        self.alloc.free(np.concatenate([req.prefix, req.reserve]))
        req.prefix = np.zeros(0, dtype=np.int64)
        req.reserve = np.zeros(0, dtype=np.int64)

    def compact(self, req: Request, kv_pool, stream=None) -> bool:
        """Gather the prefix rows into a fresh contiguous run; returns False
        (and changes nothing) when the rows already form one run or no run of
        L + headroom free slots exists."""
        L = req.length
        if L == 0 or count_runs(req.prefix) <= 1:
            return False
        run = self.alloc.alloc_run(L + self.headroom)
        if run is None:
            return False
        _gather(kv_pool, req.prefix, int(run[0]), stream)
        self.alloc.free(np.concatenate([req.prefix, req.reserve]))
        req.prefix = run[:L].copy()
        req.reserve = run[L:].copy()
        return True

    def commit_accepted(self, req: Request, tree_slots: Sequence[int], parent: Sequence[int], leaf: int,
                        kv_pool, stream=None) -> np.ndarray:
        """Append the path root..leaf of a verified tree to the request.
        Returns the slots the accepted rows now occupy."""
        tree = np.asarray(tree_slots, dtype=np.int64)
        src = tree[accepted_path(parent, leaf)]
        k = len(src)
        end = int(req.prefix[-1]) + 1 if req.length else 0
        if req.reserve.size >= k:
            dst, req.reserve = req.reserve[:k], req.reserve[k:]
        elif req.reserve.size == 0 and req.length and count_runs(req.prefix) == 1 and \
                end + k <= self.alloc.pool_slots and self.alloc.is_free[end:end + k].all():
            dst = self.alloc.take_run(end, k)
        else:
            dst = self.alloc.alloc_run(k)
        if dst is None:
            # no contiguous room anywhere: the accepted rows stay where they are
            self.alloc.free(np.setdiff1d(tree, src))
            dst = src
        else:
            _gather(kv_pool, src, int(dst[0]), stream)
            self.alloc.free(tree)
        req.prefix = np.concatenate([req.prefix, dst]).astype(np.int64)
        return dst


def _gather(kv_pool, src_slots: np.ndarray, dst_start: int, stream=None) -> None:
    """pool[dst_start : dst_start + n] = pool[src_slots] on the GPU (the
    destination rows are free slots, never among the sources)."""
    import torch
    n = int(len(src_slots))
    if n == 0:
        return
    if dst_start <= 0 or dst_start + n > kv_pool.shape[0]:
        raise ValueError("destination run outside the pool")
    if ((src_slots >= dst_start) & (src_slots < dst_start + n)).any():
        raise ValueError("destination run overlaps its sources")
    idx = torch.from_numpy(np.ascontiguousarray(src_slots, dtype=np.int32)).to(kv_pool.device)
    vb.slot_gather(kv_pool, idx, dst=kv_pool[dst_start:dst_start + n], stream=stream)
