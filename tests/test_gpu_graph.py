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


@pytest.mark.parametrize("config", [1, 2, 0])
def test_captured_step_replays_bit_identical(config):
    # 0: a 64-key prefix, whose plan is one chunk, so the captured step is a
    # single launch (the split pass writes the output)
    import torch
    log(f"[case] graph capture, workload {config}")
    if config:
        x = gen.config_inputs(config)
    else:
        x = gen.make_inputs([64], [gen.random_tree(9, np.random.default_rng(5))], 16, 4096, "scrambled", 93)
        assert vb.plan(problem(x)).max_chunks == 1
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


@pytest.mark.parametrize("cap,variants", [
    ([3000, 3000], [(3000, 3000), (1500, 2999), (0, 1), (700, 2), (3000, 0)]),
    ([5000], [(5000,), (1,), (0,), (2500,), (4097,)]),
    # a one-chunk plan: the captured step is the split pass alone, writing out
    ([60, 40], [(60, 40), (0, 1), (33, 0), (1, 40), (59, 39)]),
])
def test_one_capture_serves_changing_prefix_lengths(cap, variants):
    # VAMLA_FLAG_DEVICE_LENGTHS: lengths are read from cu_prefix / cu_tree on
    # the device and the chunk size is chosen there, so one graph captured for
    # the upper bounds replays correctly after the caller rewrites the lengths
    # and the slot list (a single request included, whose bounds otherwise come
    # from the host totals baked into the launch)
    import torch
    log(f"[case] device lengths, capacity {cap}, variants {variants}")
    rng = np.random.default_rng(len(cap))
    parents = [gen.random_tree(9, rng), gen.bounded_tree(5, rng)][:len(cap)]
    x = gen.make_inputs(cap, parents, 8, sum(cap) + 64 + 300, "scrambled", seed=90 + len(cap))
    d = to_dev(x)
    p = problem(x)
    p.flags = vb.FLAG_DEVICE_LENGTHS
    ws_g, ws_e = vb.Workspace(p), vb.Workspace(p)
    T, H = x.total_tree, x.num_heads
    out_g = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse_g = torch.empty((T, H), dtype=torch.float32, device="cuda")
    full = [x.prefix_slot_idx[x.cu_prefix[b]:x.cu_prefix[b + 1]] for b in range(x.batch)]

    def step():
        vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                           d["cu_prefix"], d["cu_tree"], ws=ws_g, out=out_g, lse=lse_g)

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

    for lens in variants:
        idx = np.concatenate([full[b][:lens[b]] for b in range(x.batch)]).astype(np.int32)
        cu_p = np.zeros(x.batch + 1, np.int32)
        cu_p[1:] = np.cumsum(lens)
        d["prefix_slot_idx"][:len(idx)].copy_(torch.from_numpy(idx))
        d["cu_prefix"].copy_(torch.from_numpy(cu_p))
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = _eager(p, d, ws_e)
        assert torch.equal(out_g.view(torch.int16), ref_out.view(torch.int16)), f"lengths {lens}: replay differs"
        assert torch.equal(lse_g, ref_lse), f"lengths {lens}: replay lse differs"
        ro, rl = vo.verify(x.q, x.pool, idx, x.tree_slot_idx, x.parent, cu_p, x.cu_tree, x.scale)
        assert_close_lse(lse_g.cpu().numpy().astype(np.float64), rl, f"lengths {lens}")
        assert_close_out(out_g.float().cpu().numpy().astype(np.float64), ro, f"lengths {lens}")
        log(f"[case] lengths {lens}: replay matches eager bit for bit and the oracle")


def test_full_size_capture_replayed_at_shorter_prefixes():
    # one graph captured for the 64k-prefix / 65-node workload with lengths
    # read on the device, replayed with the prefix cut to 40000 and 12345
    # keys: the kernels pick a smaller chunk than the host plan and must
    # still match an eager call bit for bit and the oracle (sampled heads)
    import torch
    x = gen.config_inputs(3)
    d = to_dev(x)
    p = problem(x)
    p.flags = vb.FLAG_DEVICE_LENGTHS
    ws_g, ws_e = vb.Workspace(p), vb.Workspace(p)
    T, H = x.total_tree, x.num_heads
    out_g = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse_g = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def step():
        vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                           d["cu_prefix"], d["cu_tree"], ws=ws_g, out=out_g, lse=lse_g)

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
    for L in (40000, 12345):
        log(f"[case] 64k capture replayed at prefix {L}")
        d["cu_prefix"].copy_(torch.tensor([0, L], dtype=torch.int32))
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = _eager(p, d, ws_e)
        assert torch.equal(out_g.view(torch.int16), ref_out.view(torch.int16)), f"prefix {L}: replay differs"
        assert torch.equal(lse_g, ref_lse), f"prefix {L}: replay lse differs"
        heads = [1, 8, 14]
        ro, rl = vo.verify(x.q, x.pool, x.prefix_slot_idx[:L], x.tree_slot_idx, x.parent,
                           np.array([0, L], np.int32), x.cu_tree, x.scale, heads=heads)
        got_l = lse_g.cpu().numpy().astype(np.float64)[:, heads]
        got_o = out_g.float().cpu().numpy().astype(np.float64)[:, heads]
        assert_close_lse(got_l, rl[:, heads], f"prefix {L}")
        assert_close_out(got_o, ro[:, heads], f"prefix {L}")
