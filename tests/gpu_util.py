"""Shared helpers of the GPU tests: upload seeded inputs, call the C ABI
through the binding, compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np

from speculative_decoding_tree_verify_amd import binding as vb
from speculative_decoding_tree_verify_amd import inputs as gen


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: gen.VerifyInputs):
    import torch
    dev = "cuda"

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    return dict(q=bf(x.q), kv_pool=bf(x.pool),
                prefix_slot_idx=i32(x.prefix_slot_idx) if x.total_prefix else torch.zeros(1, dtype=torch.int32, device=dev),
                tree_slot_idx=i32(x.tree_slot_idx), parent=i32(x.parent), cu_prefix=i32(x.cu_prefix),
                cu_tree=i32(x.cu_tree))


def problem(x: gen.VerifyInputs, chunk: int = 0) -> vb.Problem:
    return vb.Problem.from_host(x.cu_prefix, x.cu_tree, x.num_heads, x.pool.shape[0], x.scale, chunk=chunk)


def run_verify(x: gen.VerifyInputs, chunk: int = 0, dev=None, flags: int = 0):
    """Returns (out fp64 [T,H,512], lse fp64 [T,H]) from the HIP path."""
    import torch
    d = dev or to_dev(x)
    p = problem(x, chunk)
    p.flags = flags
    out, lse = vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                                  d["cu_prefix"], d["cu_tree"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), out


def assert_close_out(got, ref, what=""):
    """bf16 outputs: max-abs <= 1e-2, and also <= 1e-2 * max|ref| (the absolute
    bound alone is vacuous for the near-uniform softmax of small values)."""
    err = np.abs(got - ref)
    scale = np.abs(ref).max()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    tol = min(1e-2, 1e-2 * scale + 1e-6)
    log(f"[margin] {what}: out max abs err {err.max():.3e} = {err.max() / tol:.3f} of the tolerance")
    assert err.max() <= 1e-2, f"{what}: max abs err {err.max():.3e}"
    assert err.max() <= 1e-2 * scale + 1e-6, f"{what}: max abs err {err.max():.3e} vs 1e-2*max|ref|={1e-2 * scale:.3e}"


def assert_close_lse(got, ref, what=""):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite lse"
    log(f"[margin] {what}: lse max abs err {err.max():.3e} = {err.max() / 1e-3:.3f} of the tolerance")
    assert err.max() <= 1e-3, f"{what}: lse max abs err {err.max():.3e}"
