"""Graph capture of the verify step: the library enqueues plain kernel launches
on the caller's stream (no allocation, no memset, no host sync), so a captured
step replays to the eager result bit for bit.  Every replay is checked, with
eager work and synchronisations between replays, and the captured buffers
are rewritten between replays to show that a replay reads live inputs."""

import numpy as np
import pytest

import oracle.verify_oracle as vo
from speculative_decoding_tree_verify_amd import binding as vb
from speculative_decoding_tree_verify_amd import inputs as gen

from tests.gpu_util import assert_close_lse, assert_close_out, log, problem, to_dev

pytestmark = pytest.mark.gpu


def _eager(p, d, ws):
    import torch
    out, lse = vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                                  d["cu_prefix"], d["cu_tree"], ws=ws)
    torch.cuda.synchronize()
    return out.clone(), lse.clone()


@pytest.mark.parametrize("config", [1, 2])
def test_captured_step_replays_bit_identical(config):
    import torch
    log(f"[case] graph capture, workload {config}")
    x = gen.config_inputs(config)
    d = to_dev(x)
    p = problem(x)
    ws_g = vb.Workspace(p)
    ws_e = vb.Workspace(p)
    out_g = torch.empty((x.total_tree, x.num_heads, 512), dtype=torch.bfloat16, device="cuda")
    lse_g = torch.empty((x.total_tree, x.num_heads), dtype=torch.float32, device="cuda")

    def step():
        vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                           d["cu_prefix"], d["cu_tree"], ws=ws_g, out=out_g, lse=lse_g)

    # warm up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    ref_out, ref_lse = _eager(p, d, ws_e)
    q0 = d["q"].clone()
    rng = np.random.default_rng(config)
    for r in range(4):
        if r == 2:
            # new query values in the captured buffer: the replay must see them
            bits = gen.normal_bf16(rng, x.q.shape, std=0.1)
            d["q"].copy_(torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16))
            torch.cuda.synchronize()
            ref_out, ref_lse = _eager(p, d, ws_e)
            ro, rl = vo.verify(bits, x.pool, x.prefix_slot_idx, x.tree_slot_idx, x.parent, x.cu_prefix,
                               x.cu_tree, x.scale)
            assert_close_lse(ref_lse.cpu().numpy().astype(np.float64), rl, "eager after new q")
            assert_close_out(ref_out.float().cpu().numpy().astype(np.float64), ro, "eager after new q")
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        # eager work between replays, on the same device
        _ = _eager(p, d, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), ref_out.view(torch.int16)), f"replay {r}: out differs"
        assert torch.equal(lse_g, ref_lse), f"replay {r}: lse differs"
        log(f"[case] replay {r} bit-identical")
    d["q"].copy_(q0)
