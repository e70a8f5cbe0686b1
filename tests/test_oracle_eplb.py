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


def test_cleanup_worked_case_moves_then_reuses_a_hole():
    """Step 4 by hand.  E = 8 on R = 2 ranks (4 each), one spare slot per
    rank; expert 0 (rank 0) takes 10 tokens, the others 1."""
    o = EplbOracle(8, 2, window=1, threshold=1.2, max_moves=1, spare_slots=1)
    o.observe([10, 1, 1, 1, 1, 1, 1, 1])
    assert o.loads() == [13.0, 4.0]
    # migrate: expert 0 gets a copy in rank 1's spare slot (slot 4); both
    # copies serve: loads 5 + 3 = 8 and 5 + 4 = 9
    assert o.rebalance() == [(0, 1)]
    assert o.loads() == [8.0, 9.0]
    # cleanup: the copy it was taken from -- rank 0's home slot 0 -- is
    # reclaimed; expert 0 now lives on rank 1 only: loads 3 and 14
    assert o.cleanup() == [(0, 0, 0)]
    assert o.copies[0] == [1] and o.loads() == [3.0, 14.0]
    assert o.cleanup() == []                         # nothing recorded since
    off, slots, se = o.slot_map(0)
    assert se.tolist() == [-1, 1, 2, 3]              # home slot 0 stays empty
    assert slots[off[0]:off[1]].tolist() == [-1]
    off, slots, se = o.slot_map(1)
    assert se.tolist() == [4, 5, 6, 7, 0]
    assert slots[off[0]:off[1]].tolist() == [4]
    # rank 1 is now the hot one (14 / 8.5): expert 0 (10 per copy) gets a
    # copy in rank 0's spare slot; cleanup then reclaims rank 1's copy,
    # leaving a hole in its spare slot
    assert o.rebalance() == [(0, 0)]
    assert o.cleanup() == [(0, 1, 4)]
    assert o.copies[0] == [0] and o.added == [[0], [-1]]
    assert o.slot_map(0)[2].tolist() == [-1, 1, 2, 3, 0]
    assert o.slot_map(1)[2].tolist() == [4, 5, 6, 7, -1]
    # rank 1 hot (15 vs 4), but rank 0's only spare slot holds expert 0:
    # no copy can be placed
    o.observe([1, 1, 1, 1, 1, 1, 1, 12])
    assert o.loads() == [4.0, 15.0] and o.rebalance() == []
    # rank 0 hot (expert 1: 12): its copy takes rank 1's hole, slot 4
    o.observe([1, 12, 1, 1, 1, 1, 1, 1])
    assert o.loads() == [15.0, 4.0]
    assert o.rebalance() == [(1, 1)] and o.added[1] == [1]
    off, slots, se = o.slot_map(1)
    assert se.tolist() == [4, 5, 6, 7, 1] and slots[off[1]:off[2]].tolist() == [-1, 4]


def test_cleanup_keeps_the_last_copy_and_conserves_load():
    o = EplbOracle(16, 4, window=2, max_moves=2, spare_slots=2)
    rng = np.random.default_rng(11)
    p = np.ones(16)
    p[[1, 2, 9]] = 6.0
    p /= p.sum()
    for it in range(30):
        o.observe(rng.multinomial(800, p))
        o.rebalance()
        if it % 3 == 2:
            for e, r, s in o.cleanup():
                assert r not in o.copies[e]
                assert (s == e % 4 and r == e // 4) or s >= 4
        assert all(len(c) >= 1 for c in o.copies)
        assert sum(o.loads()) == pytest.approx(sum(o.window_counts()))
        for r in range(4):
            held = [e for e in range(16) if r in o.copies[e]]
            off, slots, se = o.slot_map(r)
            assert sorted(e for e in se.tolist() if e >= 0) == held
    o.pending[3][0] = True                           # expert 3's only copy
    assert len(o.copies[3]) == 1 and o.cleanup() == []
