"""fp64 CPU oracle for DDTree verify attention over an MLA latent KV pool.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package
smoke check and the benchmark's CPU-baseline leg may import or run this module;
the HIP library never calls it and shares no code with it.

What it computes (the definition, written out; no blocking, no fusion):

  For request b with prefix length L and tree of N nodes, node t, head h:
    keys   K = [pool[prefix_slot_idx[0..L)] ; pool[tree_slot_idx[0..N)]]   (L+N) x 576
    values V = K[:, :512]
    visible(t, l) = True for every prefix key l < L
    visible(t, L+j) = True  iff  j is t or an ancestor of t in the tree
    s_l   = scale * <q[t,h,:], K[l,:]>,  s_l = -inf where not visible
    lse   = log sum_l exp(s_l)
    out   = sum_l exp(s_l - lse) * V[l, :]

Sources on the pages:
  * "Mapping the Optimization Landscape for DDTree Verify Attention", section
    "Input Knowledge Required to Understand This Message", item 1: the tree
    mask lets each draft token see only its ancestors.
  * "The Architecture Detective: Uncovering FlashMLA's Potential for Blackwell
    DDTree Verification", section "The Message in Full": every tree node sees
    the whole prefix (no causal constraint among the queries over the prefix),
    RoPE is already applied, the KV layout is one latent head of width 576;
    the tree tail is attended under the mask and the two parts are merged.
  * "The Anatomy of a Kernel Investigation", section "The Message in Context":
    the correctness-first verify kernel materialises the score matrix; this
    oracle does the same, per (request, head).

Readings where the pages are silent (each is listed in the design notes):
  * a node sees itself (ancestor-or-self), which makes a chain-shaped tree
    equal to causal attention;
  * the root (node 0) is a tree node with parent -1; parents precede children;
  * V is the first 512 columns of the same 576-wide row;
  * lse is the natural log over the scaled scores;
  * a partial over zero keys is (o = 0, lse = -inf) and gets weight 0 in a merge.

Inputs are bf16 bit patterns (uint16); they are promoted exactly to fp64.
Everything else is fp64.  Parity status: pinned (brute force on every small
tree, chain == causal against torch's scaled_dot_product_attention, q = 0
closed form, planted keys, split+merge == unsplit, slot-permutation invariance).
"""

from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

D_V_DEFAULT = 512


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact promotion of bf16 bit patterns (uint16) to float64."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# the tree mask
# --------------------------------------------------------------------------

def ancestors_or_self(parent: Sequence[int], t: int) -> List[int]:
    """t, parent[t], parent[parent[t]], ..., root (request-local indices)."""
    out = []
    j = int(t)
    while j >= 0:
        out.append(j)
        j = int(parent[j])
    return out


def visibility(parent: Sequence[int], prefix_len: int) -> np.ndarray:
    """Boolean [N, L+N]: row t sees every prefix key and its ancestors-or-self."""
    n = len(parent)
    vis = np.zeros((n, prefix_len + n), dtype=bool)
    vis[:, :prefix_len] = True
    for t in range(n):
        for j in ancestors_or_self(parent, t):
            vis[t, prefix_len + j] = True
    return vis


# --------------------------------------------------------------------------
# attention over an explicit key set
# --------------------------------------------------------------------------

def attend(qrows: np.ndarray, keys: np.ndarray, scale: float, d_v: int = D_V_DEFAULT,
           vis: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of fp64 query rows [R, d] over fp64 keys [n, d].

    V = keys[:, :d_v].  `vis` ([R, n] bool) masks keys out.  Returns
    (o [R, d_v], lse [R]); rows that see no key get o = 0, lse = -inf.
    """
    R = qrows.shape[0]
    n = keys.shape[0]
    o = np.zeros((R, d_v), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if n == 0 or R == 0:
        return o, lse
    s = scale * (qrows @ keys.T)                       # [R, n] materialised scores
    if vis is not None:
        s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    if not has.any():
        return o, lse
    msafe = np.where(has, m, 0.0)
    e = np.exp(s - msafe[:, None])                      # exp(-inf) = 0 for masked keys
    den = e.sum(axis=1)
    lse = np.where(has, msafe + np.log(np.where(has, den, 1.0)), -np.inf)
    p = np.where(has[:, None], e / np.where(has, den, 1.0)[:, None], 0.0)
    o = p @ keys[:, :d_v]
    return o, lse


def merge_partials(parts: Iterable[Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Combine normalised partials (o_s, lse_s) over disjoint key sets:
    lse = log sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s.
    Partials with lse = -inf get weight 0."""
    parts = list(parts)
    if not parts:
        raise ValueError("nothing to merge")
    lses = np.stack([p[1] for p in parts], axis=0)          # [S, R]
    os_ = np.stack([p[0] for p in parts], axis=0)           # [S, R, d]
    m = lses.max(axis=0)
    has = np.isfinite(m)
    msafe = np.where(has, m, 0.0)
    w = np.exp(lses - msafe[None, :])                       # 0 for empty parts
    den = w.sum(axis=0)
    lse = np.where(has, msafe + np.log(np.where(has, den, 1.0)), -np.inf)
    wn = np.where(has[None, :], w / np.where(has, den, 1.0)[None, :], 0.0)
    o = np.einsum("sr,srd->rd", wn, os_)
    return o, lse


# --------------------------------------------------------------------------
# the verify step
# --------------------------------------------------------------------------

class Request:
    """fp64 views of one request's keys and queries."""

    def __init__(self, q_bits, pool_bits, prefix_slot_idx, tree_slot_idx, parent,
                 cu_prefix, cu_tree, b: int):
        p0, p1 = int(cu_prefix[b]), int(cu_prefix[b + 1])
        t0, t1 = int(cu_tree[b]), int(cu_tree[b + 1])
        self.L = p1 - p0
        self.N = t1 - t0
        self.t0 = t0
        self.parent = np.asarray(parent[t0:t1], dtype=np.int64)
        slots = np.concatenate([np.asarray(prefix_slot_idx[p0:p1], dtype=np.int64),
                                np.asarray(tree_slot_idx[t0:t1], dtype=np.int64)])
        self.keys = bf16_bits_to_f64(np.asarray(pool_bits)[slots])          # [L+N, d]
        self.q = bf16_bits_to_f64(np.asarray(q_bits)[t0:t1])                # [N, H, d]


def verify(q_bits, pool_bits, prefix_slot_idx, tree_slot_idx, parent, cu_prefix, cu_tree,
           scale: float, d_v: int = D_V_DEFAULT, heads: Optional[Sequence[int]] = None,
           requests: Optional[Sequence[int]] = None):
    """The full verify step: unsplit, explicitly masked attention.

    Returns (out [T, H, d_v], lse [T, H]) in fp64.  `heads` / `requests`
    restrict the work to a subset (other entries stay NaN)."""
    q_bits = np.asarray(q_bits)
    T, H = q_bits.shape[0], q_bits.shape[1]
    out = np.full((T, H, d_v), np.nan)
    lse = np.full((T, H), np.nan)
    B = len(cu_prefix) - 1
    hs = list(range(H)) if heads is None else list(heads)
    bs = list(range(B)) if requests is None else list(requests)
    for b in bs:
        r = Request(q_bits, pool_bits, prefix_slot_idx, tree_slot_idx, parent, cu_prefix, cu_tree, b)
        if r.N == 0:
            continue
        vis = visibility(r.parent, r.L)
        for h in hs:
            o, l = attend(r.q[:, h, :], r.keys, scale, d_v, vis)
            out[r.t0:r.t0 + r.N, h] = o
            lse[r.t0:r.t0 + r.N, h] = l
    return out, lse


def prefix_partial(q_bits, pool_bits, prefix_slot_idx, cu_prefix, cu_tree, b: int,
                   k0: int, k1: int, scale: float, d_v: int = D_V_DEFAULT):
    """Partial (o, lse) of every node and head of request b over prefix keys
    [k0, k1) only (no mask: every node sees every prefix key).
    Returns ([N, H, d_v], [N, H])."""
    q_bits = np.asarray(q_bits)
    p0 = int(cu_prefix[b])
    t0, t1 = int(cu_tree[b]), int(cu_tree[b + 1])
    slots = np.asarray(prefix_slot_idx[p0 + k0:p0 + k1], dtype=np.int64)
    keys = bf16_bits_to_f64(np.asarray(pool_bits)[slots])
    q = bf16_bits_to_f64(q_bits[t0:t1])
    N, H = q.shape[0], q.shape[1]
    o, l = attend(q.reshape(N * H, -1), keys, scale, d_v)
    return o.reshape(N, H, d_v), l.reshape(N, H)


def tree_partial(q_bits, pool_bits, tree_slot_idx, parent, cu_tree, b: int,
                 scale: float, d_v: int = D_V_DEFAULT):
    """Partial (o, lse) of request b over its tree keys only, under the
    ancestor-or-self mask.  Returns ([N, H, d_v], [N, H])."""
    q_bits = np.asarray(q_bits)
    t0, t1 = int(cu_tree[b]), int(cu_tree[b + 1])
    par = np.asarray(parent[t0:t1], dtype=np.int64)
    keys = bf16_bits_to_f64(np.asarray(pool_bits)[np.asarray(tree_slot_idx[t0:t1], dtype=np.int64)])
    q = bf16_bits_to_f64(q_bits[t0:t1])
    N, H = q.shape[0], q.shape[1]
    vis = visibility(par, 0)
    o = np.zeros((N, H, d_v))
    l = np.zeros((N, H))
    for h in range(H):
        oh, lh = attend(q[:, h, :], keys, scale, d_v, vis)
        o[:, h] = oh
        l[:, h] = lh
    return o, l


def gather_rows(pool_bits, idx) -> np.ndarray:
    """dst[l] = pool[idx[l]] on the raw bits (the defrag / compaction copy)."""
    return np.asarray(pool_bits)[np.asarray(idx, dtype=np.int64)].copy()
