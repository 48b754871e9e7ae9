"""VAMLA_FLAG_DEBUG_VALIDATE: the device-side check of the index data.

Bad indices used here always stay inside allocated memory, so the test is safe
even if a check were missing: out-of-range slots point into spare pool rows
past `pool_slots`, and a bad length stays within the slot list's capacity.
With the flag, a failed check leaves the split kernel without work and the
merge writing NaN; the call itself returns normally and the record names the
first violation.
"""

import numpy as np
import pytest

import oracle.verify_oracle as vo
from speculative_decoding_tree_verify_amd import binding as vb
from speculative_decoding_tree_verify_amd import inputs as gen

from tests.gpu_util import assert_close_lse, assert_close_out, log, to_dev

pytestmark = pytest.mark.gpu

SPARE = 64


def _case():
    rng = np.random.default_rng(77)
    parents = [gen.random_tree(9, rng), gen.bounded_tree(17, rng)]
    x = gen.make_inputs([300, 300], parents, 4, 2048, "scrambled", seed=77)
    return x


def _run(x, d, flags, ws=None):
    import torch
    p = vb.Problem.from_host(x.cu_prefix, x.cu_tree, x.num_heads, x.pool.shape[0], x.scale)
    p.flags = flags
    ws = ws or vb.Workspace(p)
    out, lse = vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                                  d["cu_prefix"], d["cu_tree"], ws=ws)
    torch.cuda.synchronize()
    return out, lse, vb.debug_record(p, ws), ws


def _dev_with_spare_rows(x):
    import torch
    d = to_dev(x)
    pool = torch.zeros((x.pool.shape[0] + SPARE, 576), dtype=torch.bfloat16, device="cuda")
    pool[: x.pool.shape[0]] = d["kv_pool"]
    d["kv_pool"] = pool
    return d


def test_valid_data_passes_and_matches_the_plain_call():
    x = _case()
    d = _dev_with_spare_rows(x)
    log("[case] debug validate: valid data")
    o1, l1, rec, _ = _run(x, d, vb.FLAG_DEBUG_VALIDATE)
    assert rec == (0, 0, 0)
    o0, l0, _, _ = _run(x, d, 0)
    assert np.array_equal(o1.float().cpu().numpy(), o0.float().cpu().numpy())
    assert np.array_equal(l1.cpu().numpy(), l0.cpu().numpy())
    ro, rl = vo.verify(x.q, x.pool, x.prefix_slot_idx, x.tree_slot_idx, x.parent, x.cu_prefix, x.cu_tree, x.scale)
    assert_close_lse(l1.cpu().numpy().astype(np.float64), rl, "debug validate")
    assert_close_out(o1.float().cpu().numpy().astype(np.float64), ro, "debug validate")


def _expect_rejected(x, d, flags, want):
    o, l, rec, ws = _run(x, d, flags)
    log(f"[case] record {rec}, expected {want}")
    assert rec == want
    assert np.isnan(o.float().cpu().numpy()).all()
    assert np.isnan(l.cpu().numpy()).all()
    return ws


def test_slot_past_the_pool_is_reported():
    import torch
    x = _case()
    d = _dev_with_spare_rows(x)
    P = x.pool.shape[0]
    bad = d["prefix_slot_idx"].clone()
    bad[517] = P + 3            # a spare row: inside the allocation, outside pool_slots
    bad[555] = P
    d2 = dict(d, prefix_slot_idx=bad)
    _expect_rejected(x, d2, vb.FLAG_DEBUG_VALIDATE, (-7, 2, 517))
    tbad = d["tree_slot_idx"].clone()
    tbad[20] = P + SPARE - 1
    d3 = dict(d, tree_slot_idx=tbad)
    _expect_rejected(x, d3, vb.FLAG_DEBUG_VALIDATE, (-7, 3, 20))
    # both: the prefix list comes first in the record's order
    _expect_rejected(x, dict(d, prefix_slot_idx=bad, tree_slot_idx=tbad), vb.FLAG_DEBUG_VALIDATE, (-7, 2, 517))
    torch.cuda.synchronize()


def test_bad_parent_is_reported():
    x = _case()
    d = _dev_with_spare_rows(x)
    par = d["parent"].clone()
    par[9 + 5] = 5              # request 1, node 5 names itself as parent
    _expect_rejected(x, dict(d, parent=par), vb.FLAG_DEBUG_VALIDATE, (-6, 1, 14))
    par = d["parent"].clone()
    par[9] = 0                  # request 1's root must have parent -1
    _expect_rejected(x, dict(d, parent=par), vb.FLAG_DEBUG_VALIDATE, (-6, 1, 9))


def test_length_past_max_prefix_is_reported():
    # lengths read on the device: request 0 grows past max_prefix (300) while
    # the total stays within the slot list's 600 entries
    import torch
    x = _case()
    d = _dev_with_spare_rows(x)
    d["cu_prefix"] = torch.tensor([0, 305, 505], dtype=torch.int32, device="cuda")
    _expect_rejected(x, d, vb.FLAG_DEBUG_VALIDATE | vb.FLAG_DEVICE_LENGTHS, (-8, 0, 0))


def test_a_valid_call_after_a_rejected_one_clears_the_record():
    x = _case()
    d = _dev_with_spare_rows(x)
    bad = d["tree_slot_idx"].clone()
    bad[0] = x.pool.shape[0] + 1
    ws = _expect_rejected(x, dict(d, tree_slot_idx=bad), vb.FLAG_DEBUG_VALIDATE, (-7, 3, 0))
    o, l, rec, _ = _run(x, d, vb.FLAG_DEBUG_VALIDATE, ws=ws)
    assert rec == (0, 0, 0)
    assert np.isfinite(o.float().cpu().numpy()).all() and np.isfinite(l.cpu().numpy()).all()


def test_one_launch_plan_writes_nan_on_a_bad_slot():
    # short prefixes: one chunk per request, so the split pass writes the
    # output itself; a failed check makes every element NaN there too
    import torch
    rng = np.random.default_rng(78)
    x = gen.make_inputs([40, 12], [gen.random_tree(9, rng), gen.random_tree(5, rng)], 4, 256, "scrambled", seed=78)
    p = vb.Problem.from_host(x.cu_prefix, x.cu_tree, x.num_heads, x.pool.shape[0], x.scale)
    assert vb.plan(p).max_chunks == 1
    d = _dev_with_spare_rows(x)
    o0, l0, rec, _ = _run(x, d, vb.FLAG_DEBUG_VALIDATE)
    assert rec == (0, 0, 0) and np.isfinite(o0.float().cpu().numpy()).all()
    bad = d["prefix_slot_idx"].clone()
    bad[45] = x.pool.shape[0] + 2
    _expect_rejected(x, dict(d, prefix_slot_idx=bad), vb.FLAG_DEBUG_VALIDATE, (-7, 2, 45))
    torch.cuda.synchronize()
