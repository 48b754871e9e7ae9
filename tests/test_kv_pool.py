"""CPU checks of the slot manager (kv_pool): the two free-list policies, run
searches, the Tier-0 compaction decision and the accepted-path commit's
bookkeeping.  The GPU row copy is replaced by a numpy copy on a host pool, so
every slot table the policy produces is checked against the rows it claims
to hold."""

import numpy as np
import pytest

import oracle.verify_oracle as vo
from speculative_decoding_tree_verify_amd import inputs as gen
from speculative_decoding_tree_verify_amd import kv_pool as kp


@pytest.fixture
def host_gather(monkeypatch):
    def g(pool, src, dst_start, stream=None):
        n = len(src)
        assert not ((src >= dst_start) & (src < dst_start + n)).any()
        pool[dst_start:dst_start + n] = pool[np.asarray(src)]
    monkeypatch.setattr(kp, "_gather", g)


def test_fifo_policy_is_the_pages_free_list():
    a = kp.SlotAllocator(10, "fifo")
    assert list(a.alloc(3)) == [1, 2, 3]
    a.free([2])
    assert list(a.alloc(6)) == [4, 5, 6, 7, 8, 9]
    assert list(a.alloc(1)) == [2]                   # freed slots come back last
    with pytest.raises(MemoryError):
        a.alloc(1)


def test_sorted_policy_hands_out_the_lowest_slots():
    a = kp.SlotAllocator(10, "sorted")
    x = a.alloc(5)                                   # 1..5
    a.free([x[1], x[3]])                             # 2, 4
    assert list(a.alloc(3)) == [2, 4, 6]


@pytest.mark.parametrize("policy", ["fifo", "sorted"])
def test_runs_and_bookkeeping(policy):
    rng = np.random.default_rng(0)
    a = kp.SlotAllocator(200, policy)
    held = []
    for _ in range(40):
        n = int(rng.integers(1, 12))
        if a.n_free >= n:
            held.append(a.alloc(n))
        if held and rng.random() < 0.5:
            a.free(held.pop(int(rng.integers(0, len(held)))))
    used = np.concatenate(held) if held else np.zeros(0, np.int64)
    assert len(np.unique(used)) == used.size and (used > 0).all()
    assert a.n_free == 199 - used.size
    assert (~a.is_free[used]).all() and a.is_free[1:].sum() == a.n_free
    start = a.find_run(3)
    if start is not None:
        assert a.is_free[start:start + 3].all()
        run = a.take_run(start, 3)
        assert (~a.is_free[run]).all()
        # a fifo allocation never hands out a slot a run claimed
        rest = a.alloc(a.n_free)
        assert not np.intersect1d(rest, run).size
    if used.size:
        a.free(used[:1])
        with pytest.raises(ValueError):
            a.free(used[:1])                             # double free


def test_double_free_and_padding_slot_rejected():
    a = kp.SlotAllocator(8)
    s = a.alloc(2)
    a.free(s)
    with pytest.raises(ValueError):
        a.free(s)
    with pytest.raises(ValueError):
        a.free([0])


def test_count_runs_and_path():
    assert kp.count_runs([5, 6, 7]) == 1
    assert kp.count_runs([5, 7, 8, 2]) == 3
    assert kp.count_runs([]) == 0
    parent = gen.chain_plus_branch()                 # chain 0..7, node 8 under 0
    assert kp.accepted_path(parent, 5) == [0, 1, 2, 3, 4, 5]
    assert kp.accepted_path(parent, 8) == [0, 8]
    assert kp.accepted_path(parent, 0) == [0]


def _scattered_request(pool_slots=4096, L=700, N=9, seed=3):
    rng = np.random.default_rng(seed)
    # sorted policy: the request's slots fill the holes the churn left, so
    # they scatter, while the top of the pool stays one free run
    a = kp.SlotAllocator(pool_slots, "sorted")
    churn = [a.alloc(int(rng.integers(5, 60))) for _ in range(40)]
    for j in rng.permutation(len(churn))[:25]:
        a.free(churn[j])
    prefix = a.alloc(L)
    tree = a.alloc(N)
    pool = gen.normal_bf16(rng, (pool_slots, 576))
    return a, kp.Request(prefix=prefix), tree, pool


def test_compaction_moves_rows_into_one_run(host_gather):
    a, req, tree, pool = _scattered_request()
    rows = pool[req.prefix].copy()
    # 700 rows at 1 us per 100 rows cost 7 us; a 0.1 us gain per step pays after 70 steps
    pol = kp.Tier0Defrag(a, step_gain_us=0.1, gather_us_per_row=0.01, headroom=16)
    assert kp.count_runs(req.prefix) > 1
    assert abs(pol.payback_steps(req) - 70.0) < 1e-9
    assert not pol.should_compact(req, expected_steps=69)
    assert pol.should_compact(req, expected_steps=70)
    assert not kp.Tier0Defrag(a).should_compact(req, expected_steps=1e12)   # no measured gain: never
    free_before = a.n_free
    assert pol.compact(req, pool)
    assert kp.count_runs(req.prefix) == 1
    assert np.array_equal(pool[req.prefix], rows)                   # the same rows, now contiguous
    assert req.reserve.size == 16 and req.reserve[0] == req.prefix[-1] + 1
    assert a.n_free == free_before - 16                             # old rows freed, run + reserve taken
    assert not pol.compact(req, pool)                               # already one run


def test_commit_appends_the_accepted_path(host_gather):
    a, req, tree, pool = _scattered_request()
    pol = kp.Tier0Defrag(a, headroom=4)
    pol.compact(req, pool)
    parent = gen.chain_plus_branch()
    before = pool.copy()
    L0 = req.length
    dst = pol.commit_accepted(req, tree, parent, leaf=3, kv_pool=pool)   # path 0,1,2,3: 4 rows fit the reserve
    path = [0, 1, 2, 3]
    assert np.array_equal(pool[dst], vo.gather_rows(before, tree[path]))
    assert req.length == L0 + 4 and kp.count_runs(req.prefix) == 1
    assert req.reserve.size == 0
    assert a.is_free[tree].all()                                    # every tree slot of the step is free again
    # next step: the run's end is free or not; either way the rows land in a run
    tree2 = a.alloc(9)
    dst2 = pol.commit_accepted(req, tree2, parent, leaf=8, kv_pool=pool)  # path 0, 8
    assert np.array_equal(pool[dst2], before[tree2[[0, 8]]])
    assert kp.count_runs(dst2) == 1
    assert req.length == L0 + 6
    assert a.is_free[tree2].all() and (~a.is_free[req.prefix]).all()
    assert int(a.is_free[1:].sum()) == a.n_free


def test_release_returns_every_slot(host_gather):
    a, req, tree, pool = _scattered_request()
    pol = kp.Tier0Defrag(a, headroom=8)
    pol.compact(req, pool)
    a.free(tree)
    pol.release(req)
    assert req.length == 0
    # the churn's live allocations are the only slots still taken
    assert a.n_free + int((~a.is_free[1:]).sum()) == 4095
