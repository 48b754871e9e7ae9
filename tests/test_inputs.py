"""Host-side checks of the seeded input generators."""

import numpy as np
import pytest

from speculative_decoding_tree_verify_amd import inputs as gen


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 0.1,
                        np.array([1.0, -2.5, 3.0e-5, 1.00390625, 1.01171875, 65504.0], np.float32)])
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_random_tree_is_topological():
    rng = np.random.default_rng(1)
    for n in range(1, 40):
        p = gen.random_tree(n, rng)
        assert p[0] == -1 and all(0 <= p[i] < i for i in range(1, n))


def test_bounded_tree_bounds():
    rng = np.random.default_rng(2)
    for n in (9, 33, 65):
        p = gen.bounded_tree(n, rng)
        d = gen.tree_depths(p)
        assert d.max() == min(8, n - 1)
        counts = np.bincount(p[1:], minlength=n)
        assert counts.max() <= 4
        assert all(0 <= p[i] < i for i in range(1, n))


def test_chain_plus_branch_shape():
    p = gen.chain_plus_branch()
    assert list(p) == [-1, 0, 1, 2, 3, 4, 5, 6, 0]


def test_allocator_head_alloc_tail_free():
    a = gen.FreeListAllocator(10)
    assert list(a.alloc(3)) == [1, 2, 3]          # slot 0 reserved, head of the free list
    a.free(np.array([2, 1]))
    assert list(a.alloc(6)) == [4, 5, 6, 7, 8, 9]
    assert list(a.alloc(2)) == [2, 1]              # freed slots come back in append order


def test_churned_pool_is_scrambled_and_unique():
    rng = np.random.default_rng(3)
    a = gen.churned_allocator(1 << 16, 5000, rng, n_requests=500, lo=64, hi=2048)
    s = a.alloc(5000)
    assert len(np.unique(s)) == 5000 and s.min() >= 1 and s.max() < (1 << 16)
    runs = np.count_nonzero(np.diff(s) != 1)
    assert runs > 10                                # fragmented


def test_make_inputs_logical_rows_identical_across_slot_modes():
    p = gen.chain_plus_branch()
    a = gen.make_inputs([300], [p], 4, 2048, "contiguous", seed=77)
    b = gen.make_inputs([300], [p], 4, 2048, "scrambled", seed=77)
    la = a.pool[np.concatenate([a.prefix_slot_idx, a.tree_slot_idx])]
    lb = b.pool[np.concatenate([b.prefix_slot_idx, b.tree_slot_idx])]
    assert np.array_equal(la, lb) and np.array_equal(a.q, b.q)
    assert not np.array_equal(a.prefix_slot_idx, b.prefix_slot_idx)
    used = np.zeros(2048, bool)
    used[np.concatenate([b.prefix_slot_idx, b.tree_slot_idx])] = True
    assert not used[0]
    assert np.all(b.pool[~used] == gen.BF16_NAN)


def test_config_1_shapes():
    x = gen.config_inputs(1)
    assert x.q.shape == (9, 16, 576) and x.pool.shape == (4096, 576)
    assert x.total_prefix == 1024 and x.total_tree == 9


def test_sorted_allocator_takes_the_lowest_free_slots():
    a = gen.FreeListAllocator(12, sorted=True)
    x = a.alloc(6)                       # 1..6
    assert list(x) == [1, 2, 3, 4, 5, 6]
    a.free(np.array([5, 2]))
    assert list(a.alloc(3)) == [2, 5, 7]
    assert a.size == 12 - 1 - 7


def test_sorted_churn_leaves_fewer_runs_than_the_free_list():
    # the same churn replayed with both policies: the sorted list refills holes
    # first, so a request allocated afterwards spans fewer runs
    def runs(s):
        return int(1 + np.count_nonzero(np.diff(s) != 1))
    out = {}
    for srt in (False, True):
        a = gen.churned_allocator(1 << 15, 3000, np.random.default_rng(9), n_requests=300, lo=16, hi=2048, sorted=srt)
        out[srt] = runs(a.alloc(3000))
    assert out[True] <= out[False]
    x = gen.make_inputs([2000], [gen.random_tree(9, np.random.default_rng(1))], 2, 1 << 14, "churned_sorted", seed=4,
                        churn_requests=200)
    used = np.concatenate([x.prefix_slot_idx, x.tree_slot_idx])
    assert len(np.unique(used)) == used.size and used.min() >= 1
