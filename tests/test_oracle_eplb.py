"""Pins of the EPLB-lite oracle (oracle/eplb.py), CPU only.

Expert-parallelism blog page, section 6.2 (monitor, detect at
max/mean > 1.2, copy the hottest experts of the overloaded rank) and 6.3
(redundant copies, tokens split over them).  Expected values are worked by
hand from those steps; invariants hold for any input.
"""
import numpy as np
import pytest

import oracle
from oracle.eplb import EplbOracle, bincount_experts, simulate


def test_uniform_counts_never_trigger():
    o = EplbOracle(16, 4, window=3)
    for _ in range(5):
        o.observe([7] * 16)
        assert o.imbalance() == 1.0
        assert o.rebalance() == []


def test_window_keeps_the_last_w_forwards():
    o = EplbOracle(4, 2, window=2)
    o.observe([1, 0, 0, 0])
    o.observe([0, 2, 0, 0])
    o.observe([0, 0, 3, 0])
    assert o.window_counts() == [0, 2, 3, 0]


def test_hot_expert_worked_case():
    # E = 16 on R = 4 ranks (4 experts each); expert 5 (rank 1) takes 100
    # tokens, the others 10: loads 40, 130, 40, 40, mean 62.5, ratio 2.08.
    o = EplbOracle(16, 4, window=1, threshold=1.2, max_moves=2, spare_slots=1)
    counts = [10] * 16
    counts[5] = 100
    o.observe(counts)
    assert o.loads() == [40.0, 130.0, 40.0, 40.0]
    assert o.imbalance() == pytest.approx(2.08)
    # move 1: expert 5 -> least loaded rank 0 (ties: lower rank): loads
    # 90, 80, 40, 40; move 2: rank 0 is now the most loaded, its hottest
    # copy is expert 5 (50 per copy) -> rank 2 (rank 0 has no spare left)
    assert o.rebalance() == [(5, 0), (5, 2)]
    assert o.copies[5] == [1, 0, 2]
    load = o.loads()
    assert load == pytest.approx([40 + 100 / 3, 30 + 100 / 3, 40 + 100 / 3, 40.0])


def test_threshold_is_strict():
    o = EplbOracle(4, 2, window=1, threshold=1.2)
    o.observe([30, 30, 20, 20])          # loads 60, 40: ratio exactly 1.2
    assert o.imbalance() == pytest.approx(1.2) and o.rebalance() == []
    o = EplbOracle(4, 2, window=1, threshold=1.2, max_moves=1)
    o.observe([31, 30, 20, 19])          # 61 / 50 > 1.2
    assert o.rebalance() == [(0, 1)]


def test_spare_slots_bound_the_moves():
    o = EplbOracle(8, 2, window=1, max_moves=2, spare_slots=1)
    o.observe([50, 40, 1, 1, 1, 1, 1, 1])
    # rank 0 hot: expert 0 -> rank 1; rank 1 has no spare left and rank 0 holds
    # every expert it could take a copy of, so the second move finds no target
    assert o.rebalance() == [(0, 1)]
    assert o.rebalance() == []


def test_invariants_on_random_long_tail_sequences():
    rng = np.random.default_rng(5)
    E, R = 64, 8
    hot = rng.choice(E, 12, replace=False)
    p = np.ones(E)
    p[hot] = 8.0
    p /= p.sum()
    o = EplbOracle(E, R, window=4, max_moves=2, spare_slots=2)
    for _ in range(40):
        counts = rng.multinomial(2048, p)
        o.observe(counts)
        before = o.loads()
        moves = o.rebalance()
        after = o.loads()
        assert sum(after) == pytest.approx(sum(o.window_counts()))
        if moves:
            assert max(after) <= max(before) + 1e-9
        for e in range(E):
            assert o.copies[e][0] == e // (E // R)
            assert len(set(o.copies[e])) == len(o.copies[e])
        assert all(len(a) <= 2 for a in o.added)


def test_slot_map_matches_the_placement_builder_for_one_copy():
    # one copy of expert 32 on rank 0: the section 6.3 layout the oracle's
    # placement builder writes for the replica workload
    o = EplbOracle(256, 8, window=1, spare_slots=1)
    o.copies[32].append(0)
    o.added[0].append(32)
    for rank in (0, 1, 3):
        got = o.slot_map(rank)
        ref = oracle.placement(256, 8, rank, replica_of=32 if rank == 0 else None)
        if rank == 0:
            for a, b in zip(got, ref):
                assert np.array_equal(a, b)
        else:  # other ranks see the copy on rank 0 as a second, remote entry
            off, slots, se = got
            assert np.array_equal(se, ref[2])
            home = [0] if rank == 1 else [-1]  # expert 32 lives on rank 1
            assert list(slots[off[32]:off[33]]) == home + [-1]


def test_bincount_and_simulation_smoke():
    idx = np.array([[0, 3], [3, 1]], np.int32)
    assert bincount_experts(idx, 4).tolist() == [1, 1, 0, 2]
    seq = [[10, 10, 10, 100]] * 3
    out = simulate(seq, n_experts=4, n_ranks=2, window=2, max_moves=1, spare_slots=1)
    assert out == [(0, [(3, 0)])]
