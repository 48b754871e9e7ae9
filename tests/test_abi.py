"""CPU checks of the C ABI: the library loads, exports what include/vamla.h
declares, and its host-only entry points (planning, workspace sizing,
validation, argument checks) behave without touching a GPU."""

import ctypes
import dataclasses
import math
import os
import re

import numpy as np
import pytest

from speculative_decoding_tree_verify_amd import binding as vb
from speculative_decoding_tree_verify_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vamla.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vb.LIB_PATH):
        from speculative_decoding_tree_verify_amd import build
        build.build()
    return vb.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_lists_the_entry_points():
    fns = header_functions()
    assert set(fns) == set(vb.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in header_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in vb.STATUS:
        assert L.vamla_status_string(code)
    assert L.vamla_status_string(0) == b"ok"


def prob(k):
    x = gen.config_inputs(k) if k in (1, 2) else None
    table = {
        1: vb.Problem(1, 16, 4096, gen.SOFTMAX_SCALE, 9, 9, 1024, 1024),
        2: vb.Problem(1, 16, 32768, gen.SOFTMAX_SCALE, 9, 9, 8192, 8192),
        3: vb.Problem(1, 16, 131072, gen.SOFTMAX_SCALE, 65, 65, 65536, 65536),
        4: vb.Problem(1, 128, 1 << 20, gen.SOFTMAX_SCALE, 65, 65, 131072, 131072),
        5: vb.Problem(8, 16, 1 << 21, gen.SOFTMAX_SCALE, 33, 264, 185000, 8 * 47500),
        6: vb.Problem(1, 16, 1 << 18, gen.SOFTMAX_SCALE, 1, 1, 131072, 131072),
        7: vb.Problem(1, 16, 1 << 18, gen.SOFTMAX_SCALE, 9, 9, 185000, 185000),
    }
    return table[k]


def test_hbm_bound_plans_keep_to_the_item_knee(L):
    # requests of <= 16 rows (decode) keep to 208 work items; 17 rows and up
    # are planned as before
    for prefix in (32768, 65536, 131072, 185000, 1 << 20):
        for heads in (1, 8, 16):
            info = vb.plan(vb.Problem(1, heads, 1 << 21, gen.SOFTMAX_SCALE, 1, 1, prefix, prefix))
            assert info.max_chunks <= 208, (prefix, heads, info.max_chunks)
    assert vb.plan(prob(6)).chunk == 640
    assert vb.plan(prob(7)).max_chunks * vb.plan(prob(7)).row_tiles > 208


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7])
def test_plan_covers_the_problem(L, k):
    p = prob(k)
    info = vb.plan(p)
    assert info.chunk % 32 == 0 and info.chunk >= 32
    assert info.row_tiles == math.ceil(p.max_tree * p.num_heads / 64)
    assert info.max_chunks * info.chunk >= p.max_prefix
    assert (info.max_chunks - 1) * info.chunk < max(p.max_prefix, 1)
    assert info.grid_items % 8 == 0 and info.grid_items >= p.batch * info.row_tiles * info.max_chunks
    items = p.batch * info.row_tiles * info.max_chunks
    assert info.off_part_lse >= info.off_part_o + items * 128 * 64 * 16
    assert info.workspace_bytes >= info.off_part_lse + items * 64 * 4
    assert info.workspace_bytes == vb.workspace_size(p)
    for off in (info.off_part_o, info.off_part_lse):
        assert off % 256 == 0


def test_plan_fills_the_chip_for_the_64k_config(L):
    p = prob(3)
    info = vb.plan(p)
    items = info.row_tiles * info.max_chunks
    assert 200 <= items <= 256        # one round of work items over 256 CUs
    # the last chunk also streams the tree's three 32-key tiles; it must not be the longest item
    last = p.max_prefix - (info.max_chunks - 1) * info.chunk
    assert math.ceil(last / 32) * 32 + 96 <= info.chunk


def _chunk_by_exhaustive_rule(p):
    """The chunk-size rule of the planner, evaluated over every k (the longest
    prefix split into k chunks), with the planner's cost constants."""
    cus, overhead, partial, tile, merge, hbm_items = 256, 256, 2, 32, 48, 208
    maxL = p.max_prefix
    if maxL <= tile:
        return tile
    total = p.total_prefix if p.total_prefix > 0 else maxL
    row_tiles = -(-p.max_tree * p.num_heads // 64)
    tree_keys = -(-p.max_tree // tile) * tile
    best_c, best_cost = tile, None
    for k in range(1, min(-(-maxL // tile), 8192) + 1):
        c = -(-(-(-maxL // k)) // tile) * tile
        chunks = min(-(-total // c) + -(-(p.batch - 1) // 2), p.batch * -(-maxL // c))
        items = row_tiles * chunks
        if p.max_tree * p.num_heads <= 16 and items > hbm_items and k > 1:
            continue           # HBM-bound plans keep to the item knee
        last = maxL - (-(-maxL // c) - 1) * c
        cost = -(-items // cus) * (max(c, -(-last // tile) * tile + tree_keys) + overhead)
        if c < maxL:           # partials and the merge launch; one chunk writes the output itself
            cost += items * partial + merge
        if best_cost is None or cost < best_cost or (cost == best_cost and c > best_c):
            best_c, best_cost = c, cost
    return best_c


@pytest.mark.parametrize("batch,heads,max_tree,max_prefix,total_prefix", [
    (1, 16, 65, 65536, 65536), (1, 128, 65, 131072, 131072), (8, 16, 33, 185000, 8 * 47500),
    (1, 16, 65, 4096, 4096), (64, 16, 65, 8192, 64 * 8192), (3, 16, 65, 100, 250), (1, 16, 1, 33, 33),
    (2, 128, 65, 1000003, 1500000), (5, 64, 17, 77777, 200000), (1, 16, 65, 300000, 300000),
    (1, 16, 1, 131072, 131072), (4, 16, 1, 131072, 300000), (1, 16, 9, 150, 150), (1, 16, 9, 300, 300),
])
def test_plan_chunk_matches_the_exhaustive_rule(L, batch, heads, max_tree, max_prefix, total_prefix):
    p = vb.Problem(batch, heads, 1 << 22, gen.SOFTMAX_SCALE, max_tree, max_tree * batch, max_prefix, total_prefix)
    assert vb.plan(p).chunk == _chunk_by_exhaustive_rule(p)


def test_explicit_chunk_is_kept(L):
    p = prob(2)
    p.chunk = 512
    assert vb.plan(p).chunk == 512
    p.chunk = 100                      # not a multiple of the 32-key tile
    with pytest.raises(vb.VamlaError) as e:
        vb.plan(p)
    assert e.value.status == -1


@pytest.mark.parametrize("field,value,code", [
    ("num_heads", 0, -2), ("num_heads", 129, -2), ("max_tree", 66, -2), ("max_tree", 0, -2),
    ("batch", 0, -1), ("total_tree", 0, -1), ("max_prefix", -1, -1), ("pool_slots", 0, -1),
])
def test_plan_rejects_bad_shapes(L, field, value, code):
    p = prob(1)
    setattr(p, field, value)
    with pytest.raises(vb.VamlaError) as e:
        vb.plan(p)
    assert e.value.status == code


@pytest.mark.parametrize("scale", [0.0, -0.5, float("inf"), float("nan")])
def test_plan_rejects_bad_scale(L, scale):
    p = prob(1)
    p.softmax_scale = scale
    with pytest.raises(vb.VamlaError) as e:
        vb.plan(p)
    assert e.value.status == -1


def test_plan_rejects_bad_dims(L):
    p = prob(1).params()
    p.d_qk = 512
    info = vb.VamlaPlanInfo()
    assert L.vamla_plan(ctypes.byref(p), ctypes.byref(info)) == -2
    p = prob(1).params()
    p.d_v = 576
    assert L.vamla_plan(ctypes.byref(p), ctypes.byref(info)) == -2


def test_verify_rejects_missing_workspace_before_touching_the_device(L):
    p = prob(1).params(cu_prefix_ptr=16, cu_tree_ptr=16, workspace_ptr=0, workspace_bytes=0)
    st = L.verify_attn_mla(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, None)
    assert st == -3
    need = vb.workspace_size(prob(1))
    p = prob(1).params(cu_prefix_ptr=16, cu_tree_ptr=16, workspace_ptr=256, workspace_bytes=need - 1)
    assert L.verify_attn_mla(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, None) == -3
    p = prob(1).params(cu_prefix_ptr=16, cu_tree_ptr=16, workspace_ptr=128, workspace_bytes=need)
    assert L.verify_attn_mla(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, None) == -3   # misaligned
    p = prob(1).params(cu_prefix_ptr=0, cu_tree_ptr=16, workspace_ptr=256, workspace_bytes=need)
    assert L.verify_attn_mla(ctypes.byref(p), 16, 16, 16, 16, 16, 16, 16, None) == -1


def test_slot_gather_empty_is_a_noop(L):
    assert L.vamla_slot_gather(None, None, 0, None, None) == 0
    assert L.vamla_slot_gather(None, None, -1, None, None) == -1


def test_read_rows_argument_checks(L):
    # refused before any HIP call: negative count, null pool or sink, null idx with rows
    assert L.vamla_read_rows(None, None, -1, None, None) == -1
    assert L.vamla_read_rows(None, 16, 4, 16, None) == -1
    assert L.vamla_read_rows(16, 16, 4, None, None) == -1
    assert L.vamla_read_rows(16, None, 4, 16, None) == -1


def _valid_case():
    x = gen.config_inputs(1)
    p = vb.Problem.from_host(x.cu_prefix, x.cu_tree, 16, x.pool.shape[0], gen.SOFTMAX_SCALE)
    return x, p


def test_validate_accepts_generated_inputs(L):
    x, p = _valid_case()
    assert vb.validate(p, x.parent, x.cu_tree, x.cu_prefix, x.prefix_slot_idx, x.tree_slot_idx) == 0
    x5 = gen.make_inputs([300, 0, 70], [gen.random_tree(5, np.random.default_rng(1)), np.array([-1]),
                                        gen.chain_plus_branch()], 4, 4096, "scrambled", seed=3)
    p5 = vb.Problem.from_host(x5.cu_prefix, x5.cu_tree, 4, 4096, 0.1)
    assert vb.validate(p5, x5.parent, x5.cu_tree, x5.cu_prefix, x5.prefix_slot_idx, x5.tree_slot_idx) == 0


def test_validate_catches_bad_trees(L):
    x, p = _valid_case()
    bad = x.parent.copy()
    bad[3] = 3                        # self parent
    assert vb.validate(p, bad, x.cu_tree, x.cu_prefix) == -6
    bad = x.parent.copy()
    bad[2] = 5                        # parent after child
    assert vb.validate(p, bad, x.cu_tree, x.cu_prefix) == -6
    bad = x.parent.copy()
    bad[0] = 0                        # root must be -1
    assert vb.validate(p, bad, x.cu_tree, x.cu_prefix) == -6
    bad = x.parent.copy()
    bad[4] = -1                       # second root
    assert vb.validate(p, bad, x.cu_tree, x.cu_prefix) == -6


def test_validate_catches_bad_slots_and_lengths(L):
    x, p = _valid_case()
    s = x.prefix_slot_idx.copy()
    s[10] = x.pool.shape[0]
    assert vb.validate(p, x.parent, x.cu_tree, x.cu_prefix, s, x.tree_slot_idx) == -7
    t = x.tree_slot_idx.copy()
    t[0] = -2
    assert vb.validate(p, x.parent, x.cu_tree, x.cu_prefix, x.prefix_slot_idx, t) == -7
    cp = x.cu_prefix.copy()
    cp[1] += 1
    assert vb.validate(p, x.parent, x.cu_tree, cp) == -8
    p2 = vb.Problem(**{**p.__dict__, "max_tree": 8})
    assert vb.validate(p2, x.parent, x.cu_tree, x.cu_prefix) == -1     # total_tree > batch * max_tree
    # two requests within the totals' bound, one of them past max_tree
    x2 = gen.make_inputs([10, 10], [gen.random_tree(3, np.random.default_rng(2)),
                                    gen.random_tree(7, np.random.default_rng(3))], 2, 64, "scrambled", seed=4)
    p3 = vb.Problem.from_host(x2.cu_prefix, x2.cu_tree, 2, 64, 0.1)
    assert vb.validate(p3, x2.parent, x2.cu_tree, x2.cu_prefix, x2.prefix_slot_idx, x2.tree_slot_idx) == 0
    p3.max_tree = 5
    assert vb.validate(p3, x2.parent, x2.cu_tree, x2.cu_prefix) == -8


def test_flags(L):
    # VAMLA_FLAG_DEVICE_LENGTHS and VAMLA_FLAG_DEBUG_VALIDATE are defined; neither changes the plan
    p = prob(3)
    base = vb.plan(p)
    for ok in (vb.FLAG_DEVICE_LENGTHS, vb.FLAG_DEBUG_VALIDATE, vb.FLAG_DEVICE_LENGTHS | vb.FLAG_DEBUG_VALIDATE):
        p.flags = ok
        info = vb.plan(p)
        assert (info.chunk, info.max_chunks, info.grid_items, info.workspace_bytes, info.off_debug_record) == \
            (base.chunk, base.max_chunks, base.grid_items, base.workspace_bytes, base.off_debug_record)
    for bad in (4, 8, 1 << 31, 7):
        p.flags = bad
        with pytest.raises(vb.VamlaError) as e:
            vb.plan(p)
        assert e.value.status == -1


def test_debug_record_sits_inside_the_workspace(L):
    for k in range(1, 8):
        info = vb.plan(prob(k))
        assert info.off_debug_record % 256 == 0
        assert info.off_debug_record >= info.off_part_lse
        assert info.off_debug_record + 16 <= info.workspace_bytes


@pytest.mark.parametrize("batch,max_tree,total_tree,max_prefix,total_prefix", [
    (1, 4, 9, 100, 100),        # one request with more nodes than max_tree
    (1, 9, 9, 0, 1000),         # one request with a prefix past max_prefix
    (3, 9, 28, 100, 200),       # more nodes in total than 3 requests of max_tree
    (3, 9, 27, 100, 301),       # more prefix in total than 3 requests of max_prefix
])
def test_plan_rejects_totals_beyond_the_bounds(L, batch, max_tree, total_tree, max_prefix, total_prefix):
    # chunks and row tiles are planned from the bounds: a request past them
    # would be cut short silently
    p = vb.Problem(batch, 16, 1 << 20, gen.SOFTMAX_SCALE, max_tree, total_tree, max_prefix, total_prefix)
    with pytest.raises(vb.VamlaError) as e:
        vb.plan(p)
    assert e.value.status == -1
    p.total_tree, p.total_prefix = min(total_tree, batch * max_tree), min(total_prefix, batch * max_prefix)
    vb.plan(p)


def test_binding_checks_arguments_before_any_launch(L):
    # wrong dtypes and sizes raise in the binding (CPU tensors: the checks
    # come before the device-pointer check, so nothing reaches the library)
    import torch
    x, p = _valid_case()
    T, H = x.total_tree, x.num_heads
    ok = dict(q=torch.zeros((T, H, 576), dtype=torch.bfloat16),
              kv_pool=torch.zeros((x.pool.shape[0], 576), dtype=torch.bfloat16),
              prefix_slot_idx=torch.zeros(x.total_prefix, dtype=torch.int32),
              tree_slot_idx=torch.zeros(T, dtype=torch.int32), parent=torch.zeros(T, dtype=torch.int32),
              cu_prefix=torch.tensor(x.cu_prefix), cu_tree=torch.tensor(x.cu_tree))
    out_ok = torch.zeros((T, H, 512), dtype=torch.bfloat16)
    lse_ok = torch.zeros((T, H), dtype=torch.float32)

    def call(**kw):
        a = dict(ok, **{k: v for k, v in kw.items() if k in ok})
        return vb.verify_attn_mla(p, a["q"], a["kv_pool"], a["prefix_slot_idx"], a["tree_slot_idx"], a["parent"],
                                  a["cu_prefix"], a["cu_tree"], out=kw.get("out", out_ok), lse=kw.get("lse", lse_ok))
    bad_cases = [
        dict(prefix_slot_idx=torch.zeros(x.total_prefix, dtype=torch.int64)),      # int64 read as int32 pairs
        dict(prefix_slot_idx=torch.zeros(x.total_prefix - 1, dtype=torch.int32)),  # short
        dict(tree_slot_idx=torch.zeros(T - 1, dtype=torch.int32)),
        dict(parent=torch.zeros(T, dtype=torch.int64)),
        dict(cu_prefix=torch.tensor(x.cu_prefix, dtype=torch.int64)),
        dict(cu_tree=torch.zeros(1, dtype=torch.int32)),
        dict(q=torch.zeros((T, H, 512), dtype=torch.bfloat16)),
        dict(q=torch.zeros((T, H, 576), dtype=torch.float32)),
        dict(kv_pool=torch.zeros((x.pool.shape[0] - 1, 576), dtype=torch.bfloat16)),  # fewer rows than pool_slots
        dict(kv_pool=torch.zeros((x.pool.shape[0], 512), dtype=torch.bfloat16)),
        dict(out=torch.zeros((T, H, 512), dtype=torch.float32)),
        dict(out=torch.zeros((T - 1, H, 512), dtype=torch.bfloat16)),
        dict(lse=torch.zeros((T, H), dtype=torch.bfloat16)),
        dict(lse=torch.zeros((T, H + 1), dtype=torch.float32)),
    ]
    for kw in bad_cases:
        with pytest.raises((TypeError, ValueError)) as e:
            call(**kw)
        assert "GPU" not in str(e.value), (kw, e.value)      # refused by a shape/dtype check
    with pytest.raises(ValueError, match="GPU"):                # well-formed CPU tensors reach the device check
        call()
    with pytest.raises((TypeError, ValueError)):
        vb.slot_gather(ok["kv_pool"], torch.zeros(4, dtype=torch.int64))
    with pytest.raises((TypeError, ValueError)):
        vb.slot_gather(ok["kv_pool"], torch.zeros(4, dtype=torch.int32), dst=torch.zeros((3, 576), dtype=torch.bfloat16))


def test_plan_cache_follows_every_scalar(L):
    # the library keeps the last plan per host thread, keyed by every scalar
    # field: alternating problems must each get their own plan back
    probs = [prob(1), prob(3), prob(6), prob(1)]
    fresh = []
    for p in probs:
        info = vb.plan(p)
        fresh.append((info.chunk, info.row_tiles, info.max_chunks, info.grid_items, info.workspace_bytes))
    assert fresh[0] == fresh[3] and fresh[0] != fresh[1] and fresh[1] != fresh[2]
    base = prob(3)
    a = vb.plan(base)
    changes = [dict(chunk=256), dict(num_heads=8), dict(max_tree=9, total_tree=9), dict(total_prefix=1000),
               dict(max_prefix=70000), dict(flags=vb.FLAG_DEVICE_LENGTHS)]
    for ch in changes:
        b = vb.plan(dataclasses.replace(base, **ch))
        again = vb.plan(base)
        assert (again.chunk, again.max_chunks, again.workspace_bytes) == (a.chunk, a.max_chunks, a.workspace_bytes)
        if "flags" not in ch:
            assert (b.chunk, b.row_tiles, b.max_chunks) != (a.chunk, a.row_tiles, a.max_chunks), ch


def test_binding_requires_one_device(L):
    # every tensor of a call must be on one GPU: the call runs with that
    # device current, on its stream (a tensor elsewhere would hand the
    # kernels another device's pointers)
    import types
    import torch
    on = lambda d: types.SimpleNamespace(device=torch.device(d))
    assert vb._device(on("cuda:0"), None, on("cuda:0")) == torch.device("cuda:0")
    with pytest.raises(ValueError, match="one GPU"):
        vb._device(on("cuda:0"), on("cuda:1"))
    with pytest.raises(ValueError, match="on the GPU"):
        vb._device(on("cuda:0"), on("cpu"))


def test_bench_refuses_more_than_one_gpu():
    # the path runs on one GPU; bench.py says so instead of measuring
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def test_static_entry_refuses_problems_past_its_workspace(L):
    # 64 requests of 65 nodes x 128 heads need far more than the static
    # workspace: refused on the host, before any HIP call (this runs without a GPU)
    p = vb.Problem(64, 128, 1 << 20, gen.SOFTMAX_SCALE, 65, 64 * 65, 4096, 64 * 4096)
    assert vb.workspace_size(p) > vb.STATIC_WORKSPACE_BYTES
    prm = p.params(cu_prefix_ptr=16, cu_tree_ptr=16)
    assert L.verify_attn_mla_static(ctypes.byref(prm), 16, 16, 16, 16, 16, 16, 16, None) == -9
    assert L.vamla_status_string(-9) != b"unknown status"
