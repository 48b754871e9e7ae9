"""verify_attn_mla_static (the entry point that allocates nothing) against
verify_attn_mla on the same inputs: two calls in a row, the second with a
smaller problem, each bit-identical to the caller-workspace entry point (same
kernels, same plan) and within tolerance of the oracle."""

import numpy as np
import pytest

import oracle.verify_oracle as vo
from speculative_decoding_tree_verify_amd import binding as vb
from speculative_decoding_tree_verify_amd import inputs as gen

from tests.gpu_util import assert_close_lse, assert_close_out, log, problem, to_dev

pytestmark = pytest.mark.gpu


def _both(x):
    import torch
    d = to_dev(x)
    p = problem(x)
    log(f"[case] static workspace: B={x.batch} prefix={x.total_prefix} T={x.total_tree} H={x.num_heads} "
        f"workspace {vb.workspace_size(p)} B")
    assert vb.workspace_size(p) <= vb.STATIC_WORKSPACE_BYTES
    o_s, l_s = vb.verify_attn_mla_static(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"],
                                         d["parent"], d["cu_prefix"], d["cu_tree"])
    torch.cuda.synchronize()
    o_w, l_w = vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                                  d["cu_prefix"], d["cu_tree"])
    torch.cuda.synchronize()
    assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16))
    assert torch.equal(l_s, l_w)
    ro, rl = vo.verify(x.q, x.pool, x.prefix_slot_idx, x.tree_slot_idx, x.parent, x.cu_prefix, x.cu_tree, x.scale)
    assert_close_lse(l_s.cpu().numpy().astype(np.float64), rl, "static workspace")
    assert_close_out(o_s.float().cpu().numpy().astype(np.float64), ro, "static workspace")


def test_static_workspace_matches_caller_workspace_twice():
    rng = np.random.default_rng(55)
    big = gen.make_inputs([6000, 2500], [gen.random_tree(33, rng), gen.random_tree(9, rng)], 16, 9000, "scrambled",
                          seed=55)
    small = gen.make_inputs([700], [gen.random_tree(5, rng)], 4, 1024, "scrambled", seed=56)
    _both(big)
    _both(small)
    # and a one-chunk plan, where the split pass writes the output itself
    short = gen.make_inputs([40], [gen.random_tree(9, rng)], 16, 512, "scrambled", seed=57)
    _both(short)
