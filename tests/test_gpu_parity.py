"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: bf16 out within 1e-2 max-abs and within 1e-2 * max|out_ref|;
fp32 lse within 1e-3; gather bit-exact.  Sizes span several key tiles, several
row tiles and ragged tails; the five workload configurations run at full size
(configs 4 and 5 on sampled heads / requests the oracle computes one by one).
"""

import numpy as np
import pytest

import oracle.verify_oracle as vo
from speculative_decoding_tree_verify_amd import binding as vb
from speculative_decoding_tree_verify_amd import inputs as gen

from tests.gpu_util import assert_close_lse, assert_close_out, log, problem, run_verify, to_dev

pytestmark = pytest.mark.gpu


def oracle_full(x, heads=None, requests=None):
    return vo.verify(x.q, x.pool, x.prefix_slot_idx, x.tree_slot_idx, x.parent, x.cu_prefix, x.cu_tree,
                     x.scale, heads=heads, requests=requests)


def check(x, chunk=0, heads=None, requests=None, what="", flags=0):
    log(f"[case] {what} B={x.batch} H={x.num_heads} T={x.total_tree} prefix={x.total_prefix} chunk={chunk} "
        f"flags={flags}")
    out, lse, _ = run_verify(x, chunk, flags=flags)
    ro, rl = oracle_full(x, heads, requests)
    sel = np.isfinite(rl)
    assert sel.any()
    assert_close_lse(lse[sel], rl[sel], what)
    assert_close_out(out[sel], ro[sel], what)
    return out, lse


def small(prefix_lens, parents, H, seed, pool=None, mode="scrambled", std_q=0.1):
    need = sum(prefix_lens) + sum(len(p) for p in parents)
    return gen.make_inputs(prefix_lens, parents, H, pool or (need + 257), mode, seed, std_q=std_q)


# ---------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [64, 128, 448, 0])
def test_single_request_ragged(chunk):
    rng = np.random.default_rng(1)
    x = small([1000], [gen.random_tree(9, rng)], 3, seed=11)
    check(x, chunk=chunk, what=f"ragged chunk={chunk}")


def test_several_row_tiles():
    rng = np.random.default_rng(2)
    x = small([777], [gen.random_tree(9, rng)], 16, seed=12)        # 144 rows: tiles of 64, 64, 16
    check(x, chunk=256, what="3 row tiles")


@pytest.mark.parametrize("H,N", [(1, 9), (2, 9), (5, 9), (7, 9), (16, 1), (17, 1), (4, 8), (11, 3), (16, 3),
                                 (7, 7), (8, 8), (9, 9)])
def test_partly_live_row_tile(H, N):
    # 9, 18, 45, 63, 16, 17, 32, 33, 48, 49 and 64 live rows in the only row
    # tile, and 64 + 17 in two: the MFMAs of dead 16-row halves (QK) and of
    # dead rows 32..63 (PV) are skipped; tiles of more than 16 rows stage
    # their query rows in LDS, copying only the kilobytes that hold live rows
    # (a pair with 1, 16 or 17 live rows ends inside a kilobyte)
    rng = np.random.default_rng(40 + H)
    x = small([1500], [gen.random_tree(N, rng)], H, seed=41 + H, std_q=3.0)
    check(x, chunk=256, what=f"{H * N} live rows")


def test_batch_varlen_with_empty_prefix():
    rng = np.random.default_rng(3)
    parents = [np.array([-1], np.int32), gen.random_tree(5, rng), gen.chain_plus_branch(), gen.random_tree(17, rng)]
    x = small([0, 37, 500, 1300], parents, 8, seed=13)
    check(x, chunk=192, what="batch varlen")


@pytest.mark.parametrize("flags", [0, vb.FLAG_DEVICE_LENGTHS])
@pytest.mark.parametrize("batch", [40, 70, 300])
def test_many_requests(batch, flags):
    # up to 64 requests the split kernel lists the real work items and spreads
    # them over the XCDs; past that it walks the padded item grid
    rng = np.random.default_rng(30 + batch)
    lens = [int(v) for v in rng.integers(0, 400, batch)]
    parents = [gen.random_tree(int(n), rng) for n in rng.integers(1, 10, batch)]
    x = small(lens, parents, 2, seed=31 + batch)
    check(x, chunk=128, what=f"{batch} requests", flags=flags)


def test_single_request_bounds_match_the_batched_path():
    # one request takes its bounds from the call's totals, a batch reads
    # cu_prefix / cu_tree: with the same chunk the request's partials and
    # merge are the same arithmetic, so its rows must agree bit for bit
    rng = np.random.default_rng(8)
    par_a, par_b = gen.random_tree(9, rng), gen.random_tree(5, rng)
    both = small([900, 333], [par_a, par_b], 4, seed=20)
    check(both, chunk=128, what="two requests")
    one = gen.VerifyInputs(q=both.q[:9].copy(), pool=both.pool, prefix_slot_idx=both.prefix_slot_idx[:900].copy(),
                           tree_slot_idx=both.tree_slot_idx[:9].copy(), parent=both.parent[:9].copy(),
                           cu_prefix=np.array([0, 900], np.int32), cu_tree=np.array([0, 9], np.int32),
                           num_heads=both.num_heads, scale=both.scale)
    out1, lse1, _ = run_verify(one, 128)
    out2, lse2, _ = run_verify(both, 128)
    assert np.array_equal(lse1, lse2[:9])          # fp32 values, widened exactly
    assert np.array_equal(out1, out2[:9])          # bf16 values, widened exactly
    ro, rl = oracle_full(one)
    assert_close_lse(lse1, rl, "one request")
    assert_close_out(out1, ro, "one request")


def test_no_prefix_at_all():
    rng = np.random.default_rng(4)
    x = small([0, 0], [gen.random_tree(7, rng), gen.random_tree(3, rng)], 4, seed=14)
    check(x, what="no prefix")


def test_deepest_chain_and_widest_tree():
    x = small([200], [np.arange(-1, 64, dtype=np.int32)], 2, seed=15)               # depth 64
    check(x, chunk=64, what="chain of 65")
    star = np.zeros(65, np.int32)
    star[0] = -1
    x = small([130], [star], 2, seed=16)                                              # 64 leaves
    check(x, chunk=64, what="star of 65")


def test_all_128_heads():
    rng = np.random.default_rng(5)
    x = small([300], [gen.random_tree(9, rng)], 128, seed=17)
    check(x, chunk=128, what="H=128")


def test_zero_queries_average_the_visible_values():
    # every score is 0, so each row's weights are uniform over its visible
    # keys (the prefix plus its ancestors-or-self): out is their mean V and
    # lse = ln(count).  The split kernel's reference then sits 40 log2 units
    # above every score, so each weight is 2^-40 before normalisation
    rng = np.random.default_rng(9)
    parent = gen.random_tree(9, rng)
    x = small([3000], [parent], 4, seed=92)
    x.q[:] = 0
    out, lse = check(x, chunk=1024, what="zero queries")
    depth = gen.tree_depths(parent)
    want = np.log(3000 + depth + 1.0)
    np.testing.assert_allclose(lse, np.repeat(want[:, None], 4, axis=1), atol=1e-4)


def test_sharp_scores_move_the_reference():
    rng = np.random.default_rng(6)
    x = small([3000], [gen.random_tree(9, rng)], 4, seed=18, std_q=10.0)              # score sd ~ 1.7
    check(x, chunk=1024, what="sharp scores")


def test_wide_score_spread_keeps_the_first_reference():
    # query sd 80: score sd ~ 14 nats, so within a 1024-key chunk some rows
    # climb 30-45 nats above their first tile's max.  The split kernel's
    # reference sits a fixed margin above that max with headroom on top
    # (66.5 nats in all), so no chunk restarts and every row matches
    rng = np.random.default_rng(8)
    x = small([3000], [gen.random_tree(9, rng)], 4, seed=20, std_q=80.0)
    qm = vo.bf16_bits_to_f64(x.q).reshape(-1, 576)
    km = vo.bf16_bits_to_f64(x.pool[x.prefix_slot_idx])
    s = qm @ km.T * x.scale
    jump = max((s[:, c:c + 1024].max(1) - s[:, c:c + 32].max(1)).max() for c in range(0, 3000, 1024))
    log(f"[case] largest climb over a chunk's first tile: {jump:.1f} nats")
    assert 30.0 < jump < 60.0
    _, _, restarts = check_debug(x, 1024, "score sd 14 nats")
    assert restarts == 0


@pytest.mark.parametrize("H,N,node,head", [(2, 5, 2, 1), (5, 9, 8, 4)])
@pytest.mark.parametrize("chunk", [2048, 32])
def test_reference_jump_mid_chunk(chunk, H, N, node, head):
    # one prefix key deep inside a chunk gets a score far above everything
    # before it, so the chunk's softmax reference has to move mid-chunk; with
    # 32-key chunks the key sits in chunk 46 of 63, and the merge's fold over
    # chunk lanes and waves has to move its max too.  10 and 45 live rows:
    # the row with the jump sits in a tile with dead 16-row halves (row 44
    # is in the second row pair, whose upper half is dead)
    rng = np.random.default_rng(7)
    x = small([2000], [gen.random_tree(N, rng)], H, seed=19)
    key = 1500
    slot = x.prefix_slot_idx[key]
    k = vo.bf16_bits_to_f64(x.pool[slot])
    # score ~ 250*|k|^2*scale ~ 105 nats above the rest: past the split
    # kernel's 66.5 nats of tolerance above a chunk's first key tile, so with
    # 2048-key chunks the chunk restarts
    x.q[node, head] = gen.f32_to_bf16_bits((k * 250.0).astype(np.float32))
    out, lse, restarts = check_debug(x, chunk, f"reference jump chunk={chunk} rows={H * N} node={node} head={head}")
    np.testing.assert_allclose(out[node, head], k[:512], atol=2e-2)
    if chunk == 2048:
        assert restarts >= 1


def check_debug(x, chunk, what):
    """check() through a call with VAMLA_FLAG_DEBUG_VALIDATE; also returns the
    split pass's restart count."""
    import torch
    log(f"[case] {what} (debug record)")
    p = problem(x, chunk)
    p.flags = vb.FLAG_DEBUG_VALIDATE
    d = to_dev(x)
    ws = vb.Workspace(p)
    o, l = vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                              d["cu_prefix"], d["cu_tree"], ws=ws)
    torch.cuda.synchronize()
    rec = vb.debug_record(p, ws, with_restarts=True)
    assert rec[:3] == (0, 0, 0)
    out, lse = o.float().cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)
    ro, rl = oracle_full(x)
    assert_close_lse(lse, rl, what)
    assert_close_out(out, ro, what)
    return out, lse, rec[3]


def test_repeated_restarts_leave_other_rows_exact():
    # one row meets keys whose scores climb by ~105 nats at a time inside one
    # 2048-key chunk (key 100 and its copy at 300, then 2x, 3x, 4x it): four
    # restarts of the chunk.  Every other row of the tile
    # (same row pair included) keeps a reference at or below its own max plus
    # the fixed margin, so all rows still match the oracle, and the climbing
    # row ends on the last key.  The tile's 36 rows are staged in LDS by the
    # prologue; a restart keeps them in registers (their ring slots are
    # refilled by then)
    rng = np.random.default_rng(70)
    H, N, node, head = 4, 9, 3, 2
    x = small([2000], [gen.random_tree(N, rng)], H, seed=71)
    k = vo.bf16_bits_to_f64(x.pool[x.prefix_slot_idx[100]])
    x.q[node, head] = gen.f32_to_bf16_bits((k * 250.0).astype(np.float32))
    for g, pos in enumerate((300, 700, 1100, 1500), start=1):
        x.pool[x.prefix_slot_idx[pos]] = gen.f32_to_bf16_bits((k * g).astype(np.float32))
    out, lse, restarts = check_debug(x, 2048, "four climbing keys in one chunk")
    assert restarts >= 4
    np.testing.assert_allclose(out[node, head], 4 * k[:512], atol=4e-2)


def test_config1():
    check(gen.config_inputs(1), what="config 1")


def test_config2_contiguous_and_scrambled_bit_identical():
    a = gen.config_inputs(2, slot_mode="contiguous")
    b = gen.config_inputs(2, slot_mode="scrambled")
    oa, la = check(a, what="config 2 contiguous")
    ob, lb = check(b, what="config 2 scrambled")
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_config3_full():
    x = gen.config_inputs(3)
    check(x, what="config 3")


def test_config3_lengths_on_the_device():
    # the chunk size is chosen in the kernels from cu_prefix (the 65536-key
    # prefix over the plan's chunk slots), not taken from the host plan
    x = gen.config_inputs(3)
    info = vb.plan(problem(x))
    dev_chunk = max(32, -(-(-(-65536 // info.max_chunks)) // 32) * 32)
    log(f"config 3 host chunk {info.chunk}, device chunk {dev_chunk}, {info.max_chunks} chunk slots")
    check(x, heads=[0, 6, 15], what="config 3, lengths on the device", flags=vb.FLAG_DEVICE_LENGTHS)


def test_config3_planted_tree_keys():
    # at full size one wrong tree key moves lse by ~1/65601, far below the
    # lse bound; a planted key makes the mask visible: a node whose query is
    # a large multiple of an ancestor's key must output that key's V row,
    # one planted on a key it must not see must not
    x = gen.config_inputs(3)
    par = x.parent
    depth = gen.tree_depths(par)
    deep = [int(t) for t in np.argsort(-depth)[:3]]
    planted = {}
    for i, t in enumerate(deep):
        anc = vo.ancestors_or_self(par, t)
        j = anc[len(anc) // 2]                       # a visible ancestor, not the node itself
        hidden = next(u for u in range(len(par)) if u not in anc)
        h_vis, h_hid = (3 * i) % 16, (3 * i + 7) % 16
        kv = vo.bf16_bits_to_f64(x.pool[x.tree_slot_idx[j]])
        kh = vo.bf16_bits_to_f64(x.pool[x.tree_slot_idx[hidden]])
        x.q[t, h_vis] = gen.f32_to_bf16_bits((kv * 40.0).astype(np.float32))
        x.q[t, h_hid] = gen.f32_to_bf16_bits((kh * 40.0).astype(np.float32))
        planted[t] = (h_vis, kv, h_hid, kh)
    heads = sorted({h for v in planted.values() for h in (v[0], v[2])})
    out, lse = check(x, heads=heads, what="config 3, planted tree keys")
    for t, (h_vis, kv, h_hid, kh) in planted.items():
        np.testing.assert_allclose(out[t, h_vis], kv[:512], atol=2e-2)
        assert np.abs(out[t, h_hid] - kh[:512]).max() > 0.1


def test_config4_sampled_heads():
    x = gen.config_inputs(4)
    check(x, heads=[0, 77, 127], what="config 4 heads 0,77,127")


def test_config5_sampled_requests():
    x = gen.config_inputs(5)
    log(f"config 5 prefix lengths {[x.prefix_len(b) for b in range(8)]}")
    check(x, requests=[0, 3, 7], heads=[0, 9, 15], what="config 5 requests 0,3,7")


def test_config5_other_requests():
    # every request of the batch meets the oracle: 1, 2, 4, 5, 6 on two heads each
    x = gen.config_inputs(5)
    check(x, requests=[1, 2, 4, 5, 6], heads=[4, 11], what="config 5 requests 1,2,4,5,6")


def test_small_rows_decode_full():
    x = gen.config_inputs(6)
    check(x, what="decode 16 rows, 131072-token prefix")


def test_small_rows_decode_batch():
    # four decode requests (one node each, 16 heads) with unequal long
    # prefixes in one churned pool: the plan keeps to the HBM-bound item cap
    # (fewer, longer chunks) and the merge folds each request's own chunks
    rng = np.random.default_rng(77)
    lens = [131072, 70001, 33000, 5]
    x = small(lens, [np.array([-1], np.int32)] * 4, 16, seed=78, pool=1 << 19, mode="churned")
    info = vb.plan(problem(x))
    log(f"[case] decode batch {lens}: chunk {info.chunk}, {info.max_chunks} chunks per request")
    assert info.max_chunks <= 208
    check(x, what="decode batch of four")


def test_small_rows_nine_queries_full():
    x = gen.config_inputs(7)
    check(x, what="9 nodes x 16 heads, 185000-token prefix")


def test_determinism():
    x = gen.config_inputs(1)
    d = to_dev(x)
    o1, l1, _ = run_verify(x, dev=d)
    o2, l2, _ = run_verify(x, dev=d)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# --- stage-level parity ----------------------------------------------------

@pytest.mark.parametrize("lens,chunk", [([700, 250, 0], 256), ([128, 64, 0], 64)])
def test_stage_split_partials(lens, chunk):
    # chunk partials on their own: every chunk but a request's last covers its
    # prefix keys only; the last one (chunk 0 with no prefix) also the tree keys
    # under the ancestor mask, which is the oracle's prefix and tree partials merged
    import torch
    rng = np.random.default_rng(8)
    parents = [gen.random_tree(9, rng), gen.bounded_tree(33, rng), gen.random_tree(65, rng)]
    x = small(lens, parents, 8, seed=20)
    p = problem(x, chunk=chunk)
    d = to_dev(x)
    ws = vb.Workspace(p)
    log(f"[case] split partials lens={lens} chunk={chunk}")
    vb.split_partials(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                      d["cu_prefix"], d["cu_tree"], ws)
    torch.cuda.synchronize()
    v = vb.workspace_views(p, ws)
    part_o = v["part_o"].cpu().numpy()
    part_lse = v["part_lse"].cpu().numpy()
    for b in range(x.batch):
        L, N, H = x.prefix_len(b), x.tree_len(b), x.num_heads
        S = max(1, -(-L // chunk))
        for s in range(S):
            parts = []
            if L:
                parts.append(vo.prefix_partial(x.q, x.pool, x.prefix_slot_idx, x.cu_prefix, x.cu_tree, b,
                                               s * chunk, min(L, (s + 1) * chunk), x.scale))
            if s == S - 1:
                parts.append(vo.tree_partial(x.q, x.pool, x.tree_slot_idx, x.parent, x.cu_tree, b, x.scale))
            ro, rl = vo.merge_partials([(o.reshape(N * H, 512), l.reshape(N * H)) for o, l in parts])
            rows = np.arange(N * H)
            tile, rit = rows // 64, rows % 64
            got_l = part_lse[b, tile, s, rit]
            got_o = part_o[b, tile, s].reshape(len(rows), 128, 64, 4)[np.arange(len(rows)), :, rit, :].reshape(len(rows), 512)
            assert_close_lse(got_l, rl, f"partial b={b} s={s}")
            np.testing.assert_allclose(got_o, ro, atol=2e-3 * np.abs(ro).max() + 1e-6)


@pytest.mark.parametrize("lens,N,H", [([64], 9, 16), ([0, 37, 64, 5], 5, 8), ([128], 65, 16), ([31], 33, 128)])
def test_one_launch_for_single_chunk_plans(lens, N, H):
    # short prefixes plan one chunk per request: the split pass writes out and
    # lse itself (one launch).  A merge of one partial is the identity, so the
    # result equals the two stage entry points' bit for bit on the same plan,
    # and it meets the oracle
    import torch
    rng = np.random.default_rng(60 + N)
    x = small(lens, [gen.random_tree(N, rng) for _ in lens], H, seed=61 + N)
    p = problem(x)
    info = vb.plan(p)
    log(f"[case] one launch lens={lens} N={N} H={H}: chunk {info.chunk}, {info.max_chunks} chunk(s)")
    assert info.max_chunks == 1
    d = to_dev(x)
    ws = vb.Workspace(p)
    o1, l1 = vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                                d["cu_prefix"], d["cu_tree"], ws=ws)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    vb.split_partials(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                      d["cu_prefix"], d["cu_tree"], ws)
    vb.lse_merge(p, d["cu_prefix"], d["cu_tree"], ws, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    ro, rl = oracle_full(x)
    assert_close_lse(l1.cpu().numpy().astype(np.float64), rl, "one launch")
    assert_close_out(o1.float().cpu().numpy().astype(np.float64), ro, "one launch")


def test_slot_gather_bit_exact():
    import torch
    x = gen.config_inputs(2, slot_mode="scrambled")
    d = to_dev(x)
    idx = d["prefix_slot_idx"]
    dst = vb.slot_gather(d["kv_pool"], idx)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, vo.gather_rows(x.pool, x.prefix_slot_idx))
    # ragged count, repeated slots
    idx2 = torch.tensor([5, 5, 1, 32767, 9, 9, 9], dtype=torch.int32, device="cuda")
    dst2 = vb.slot_gather(d["kv_pool"], idx2)
    torch.cuda.synchronize()
    assert np.array_equal(dst2.view(torch.int16).cpu().numpy().view(np.uint16),
                          vo.gather_rows(x.pool, [5, 5, 1, 32767, 9, 9, 9]))


def test_read_rows_checksum():
    # the XOR of the sink words equals the XOR of every 32-bit word of the
    # rows named, for a workload's prefix, a ragged repeated list and none
    import torch
    x = gen.config_inputs(2, slot_mode="scrambled")
    d = to_dev(x)
    words = lambda rows: np.bitwise_xor.reduce(np.ascontiguousarray(rows).view(np.uint32), axis=None)
    for idx_h in (x.prefix_slot_idx, np.array([5, 5, 1, 32767, 9, 9, 9], np.int32)):
        sink = vb.read_rows(d["kv_pool"], torch.from_numpy(np.ascontiguousarray(idx_h, np.int32)).cuda())
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == words(vo.gather_rows(x.pool, idx_h)), len(idx_h)
    sink = vb.read_rows(d["kv_pool"], torch.zeros(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert not sink.cpu().numpy().any()


def test_defragmented_pool_gives_identical_result():
    import torch
    x = gen.config_inputs(2, slot_mode="scrambled")
    d = to_dev(x)
    o1, l1, _ = run_verify(x, dev=d)
    # compact prefix then tree rows into slots 1..n of a fresh pool via the gather kernel
    order = torch.cat([d["prefix_slot_idx"], d["tree_slot_idx"]])
    rows = vb.slot_gather(d["kv_pool"], order)
    pool2 = torch.zeros_like(d["kv_pool"])
    pool2[1:1 + rows.shape[0]] = rows
    n = x.total_prefix
    d2 = dict(d, kv_pool=pool2,
              prefix_slot_idx=torch.arange(1, n + 1, dtype=torch.int32, device="cuda"),
              tree_slot_idx=torch.arange(n + 1, n + 1 + x.total_tree, dtype=torch.int32, device="cuda"))
    o2, l2, _ = run_verify(x, dev=d2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_rows_beyond_4gib_of_pool():
    # Every row the step reads sits past byte 2^32 of a 4.6 GB pool whose other
    # rows are NaN: addressing that lost the high bits of slot * 1152 would
    # land inside the pool on a NaN row.
    import torch
    rng = np.random.default_rng(10)
    x = small([700, 130], [gen.random_tree(9, rng), gen.chain_plus_branch()], 8, seed=22)
    big = 4_000_000
    base = (1 << 32) // 1152 + 1000
    used = np.concatenate([x.prefix_slot_idx, x.tree_slot_idx]).astype(np.int64)
    uniq = np.unique(used)
    remap = np.full(x.pool.shape[0], -1, np.int64)
    remap[uniq] = base + rng.permutation(len(uniq))
    assert remap[uniq].max() < big
    d = to_dev(x)
    pool = torch.full((big, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    pool[torch.from_numpy(remap[uniq]).cuda()] = d["kv_pool"][torch.from_numpy(uniq).cuda()]
    d = dict(d, kv_pool=pool,
             prefix_slot_idx=torch.from_numpy(remap[x.prefix_slot_idx].astype(np.int32)).cuda(),
             tree_slot_idx=torch.from_numpy(remap[x.tree_slot_idx].astype(np.int32)).cuda())
    log(f"[case] pool of {big} slots, rows at slots >= {base}")
    p = vb.Problem.from_host(x.cu_prefix, x.cu_tree, x.num_heads, big, x.scale, chunk=256)
    out, lse = vb.verify_attn_mla(p, d["q"], d["kv_pool"], d["prefix_slot_idx"], d["tree_slot_idx"], d["parent"],
                                  d["cu_prefix"], d["cu_tree"])
    torch.cuda.synchronize()
    ro, rl = oracle_full(x)
    assert_close_lse(lse.cpu().numpy().astype(np.float64), rl, "beyond 4 GiB")
    assert_close_out(out.float().cpu().numpy().astype(np.float64), ro, "beyond 4 GiB")
    del pool
    torch.cuda.empty_cache()


def _sweep_case(i):
    """Seeded random shape i of the sweep: 1-5 requests, 1-128 heads, trees of
    1-65 nodes (random, bounded-depth or chains), prefixes from empty to 2500
    keys with ragged ends, an explicit or planned chunk, a query spread from
    near-uniform softmax to ~14 nats, and any slot layout."""
    rng = np.random.default_rng(9000 + i)
    B = int(rng.integers(1, 6))
    H = int(rng.choice([1, 2, 3, 5, 8, 16, 32, 128]))
    n_max = 65 if H <= 16 else 9                       # keep the oracle's work small at 128 heads
    parents = []
    for _ in range(B):
        n = int(rng.integers(1, n_max + 1))
        kind = rng.integers(3)
        if kind == 0:
            parents.append(gen.random_tree(n, rng))
        elif kind == 1:
            parents.append(gen.bounded_tree(n, rng))
        else:
            parents.append(np.arange(-1, n - 1, dtype=np.int32))   # a chain
    lens = [int(v) for v in rng.choice([0, 1, 31, 32, 33, 95, 400, 777, 1500, 2500], B)]
    chunk = int(rng.choice([0, 0, 32, 64, 96, 224, 512]))
    std_q = float(rng.choice([0.1, 3.0, 30.0]))
    mode = str(rng.choice(["scrambled", "contiguous", "churned"]))
    need = sum(lens) + sum(len(p) for p in parents)
    pool = need + 257 if mode != "churned" else need + 20000   # churn allocates up to 16384 slots at once
    x = gen.make_inputs(lens, parents, H, pool, mode, seed=9100 + i, std_q=std_q, churn_requests=200)
    return x, chunk, f"sweep {i}: B={B} H={H} N={[len(p) for p in parents]} L={lens} chunk={chunk} std_q={std_q} {mode}"


@pytest.mark.parametrize("i", range(48))
def test_random_shape_sweep(i):
    # every third case reads the request lengths on the device
    x, chunk, what = _sweep_case(i)
    flags = vb.FLAG_DEVICE_LENGTHS if i % 3 == 2 else 0
    check(x, chunk=chunk, what=what, flags=flags)
