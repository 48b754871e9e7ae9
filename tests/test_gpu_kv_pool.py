"""Tier-0 compaction and the accepted-path commit on the GPU.

A request's prefix rows are scattered over a churned pool; the policy moves
them into one run with vamla_slot_gather, then a verify step's accepted path
is committed next to that run.  Checks: moved rows equal oracle.gather_rows of
the old slots bit for bit; a verify on the moved layout is bit-identical to
the verify before the move (slots vacated by the move are NaN-poisoned, so a
stale slot would show); the next step over the extended prefix matches the
oracle.
"""

import numpy as np
import pytest

import oracle.verify_oracle as vo
from speculative_decoding_tree_verify_amd import binding as vb
from speculative_decoding_tree_verify_amd import inputs as gen
from speculative_decoding_tree_verify_amd import kv_pool as kp

from tests.gpu_util import assert_close_lse, assert_close_out, log

pytestmark = pytest.mark.gpu

H = 8
P = 16384


def _verify(pool_t, q_bits, prefix, tree, parent):
    import torch
    dev = "cuda"
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    q = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    cu_p = np.array([0, len(prefix)], np.int32)
    cu_t = np.array([0, len(tree)], np.int32)
    prob = vb.Problem.from_host(cu_p, cu_t, H, P, gen.SOFTMAX_SCALE)
    out, lse = vb.verify_attn_mla(prob, q, pool_t, i32(prefix), i32(tree), i32(parent), i32(cu_p), i32(cu_t))
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()


def test_compaction_and_commit_keep_results_and_rows():
    import torch
    rng = np.random.default_rng(123)
    alloc = kp.SlotAllocator(P, "sorted")
    churn = [alloc.alloc(int(rng.integers(8, 200))) for _ in range(60)]
    for j in rng.permutation(len(churn))[:40]:
        alloc.free(churn[j])
    req = kp.Request(prefix=alloc.alloc(3000))
    parent = gen.chain_plus_branch()
    tree = alloc.alloc(len(parent))
    log(f"[case] prefix of {req.length} rows in {kp.count_runs(req.prefix)} runs")
    assert kp.count_runs(req.prefix) > 5

    host = np.full((P, 576), gen.BF16_NAN, dtype=np.uint16)
    used = np.concatenate([req.prefix, tree])
    host[used] = gen.normal_bf16(rng, (used.size, 576))
    q = gen.normal_bf16(rng, (len(parent), H, 576), std=3.0)
    pool_t = torch.from_numpy(host.view(np.int16)).cuda().view(torch.bfloat16)
    out0, lse0 = _verify(pool_t, q, req.prefix, tree, parent)

    # Tier-0 compaction: one run, vacated slots poisoned, bit-identical result
    pol = kp.Tier0Defrag(alloc, step_gain_us=1.0, headroom=32)
    old_prefix = req.prefix.copy()
    assert pol.should_compact(req, expected_steps=1000)
    assert pol.compact(req, pool_t)
    torch.cuda.synchronize()
    assert kp.count_runs(req.prefix) == 1
    moved = pool_t[torch.from_numpy(req.prefix).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(moved, vo.gather_rows(host, old_prefix))
    pool_t[torch.from_numpy(old_prefix).cuda()] = float("nan")
    out1, lse1 = _verify(pool_t, q, req.prefix, tree, parent)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)

    # accepted path 0..5 committed into the reserve after the run
    leaf = 5
    path = kp.accepted_path(parent, leaf)
    dst = pol.commit_accepted(req, tree, parent, leaf, pool_t)
    torch.cuda.synchronize()
    assert kp.count_runs(req.prefix) == 1 and req.length == 3000 + len(path)
    got = pool_t[torch.from_numpy(dst).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, vo.gather_rows(host, tree[path]))
    # the same step over the committed layout (path nodes read from their new
    # slots) is bit-identical to the step before the commit
    tree_moved = tree.copy()
    tree_moved[path] = dst
    out2, lse2 = _verify(pool_t, q, req.prefix[:3000], tree_moved, parent)
    assert np.array_equal(out0, out2) and np.array_equal(lse0, lse2)

    # next step over the extended prefix, against the oracle
    host2 = pool_t.view(torch.int16).cpu().numpy().view(np.uint16).copy()
    parent2 = gen.random_tree(9, rng)
    tree2 = alloc.alloc(9)
    rows2 = gen.normal_bf16(rng, (9, 576))
    host2[tree2] = rows2
    pool_t[torch.from_numpy(tree2).cuda()] = torch.from_numpy(rows2.view(np.int16)).cuda().view(torch.bfloat16)
    q2 = gen.normal_bf16(rng, (9, H, 576), std=3.0)
    out3, lse3 = _verify(pool_t, q2, req.prefix, tree2, parent2)
    ro, rl = vo.verify(q2, host2, req.prefix.astype(np.int32), tree2.astype(np.int32), parent2,
                       np.array([0, req.length], np.int32), np.array([0, 9], np.int32), gen.SOFTMAX_SCALE)
    o3 = out3.astype(np.uint32) << 16
    assert_close_lse(lse3.astype(np.float64), rl, "step after commit")
    assert_close_out(o3.view(np.float32).astype(np.float64), ro, "step after commit")
