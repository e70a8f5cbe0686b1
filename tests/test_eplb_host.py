"""EPLB-lite host planner in libmoe against the oracle (CPU only).

The monitor, trigger, greedy replica planner and per-rank slot tables of
libmoe (moe_eplb_*, host code) must make the same decisions as the oracle
(oracle/eplb.py) on the same count sequences: loads and the imbalance ratio
bit-identical (both accumulate count/n_copies in expert order in double),
the same moves in the same order, the same slot tables for every rank.
"""
import numpy as np
import pytest

from oracle.eplb import EplbOracle

moe = pytest.importorskip("expert_router_gemm_amd")


def _pair(E, R, W, moves, spare, thr=1.2):
    cfg = moe.make_eplb_config(n_experts=E, n_ranks=R, window=W, max_moves=moves,
                               spare_slots=spare, threshold=thr)
    st = np.zeros(moe.moe_eplb_state_bytes(cfg), np.uint8)
    moe.moe_eplb_init(cfg, st)
    return cfg, st, EplbOracle(E, R, window=W, threshold=thr, max_moves=moves, spare_slots=spare)


def _run(seq, E, R, W, moves, spare, thr=1.2, cleanup_every=0):
    cfg, st, o = _pair(E, R, W, moves, spare, thr)
    n_moves = 0
    for i, counts in enumerate(seq):
        if cleanup_every and i % cleanup_every == cleanup_every - 1:
            assert moe.moe_eplb_cleanup(st, cfg) == o.cleanup()
        counts = np.ascontiguousarray(counts, np.int32)
        moe.moe_eplb_observe(st, counts)
        o.observe(counts)
        loads, imb = moe.moe_eplb_loads(st, R)
        assert loads.tolist() == o.loads()
        assert imb == o.imbalance()
        got = moe.moe_eplb_rebalance(st, moves)
        ref = o.rebalance()
        assert got == ref
        n_moves += len(got)
        for rank in range(R):
            a = moe.moe_eplb_slot_map(st, cfg, rank)
            b = o.slot_map(rank)
            for x, y in zip(a, b):
                assert np.array_equal(x, y)
    return n_moves


@pytest.mark.parametrize("seed", range(6))
def test_planner_matches_oracle_on_long_tail_sequences(seed):
    rng = np.random.default_rng(seed)
    E, R = [(256, 8), (64, 8), (16, 4), (32, 2), (256, 8), (128, 16)][seed]
    hot = rng.choice(E, max(1, int(0.3 * E)), replace=False)
    p = np.ones(E)
    p[hot] = rng.uniform(2, 8)
    p[: E // R] *= 2.0  # rank 0's experts run hot: the trigger fires
    p /= p.sum()
    seq = [rng.multinomial(int(rng.integers(100, 5000)), p) for _ in range(30)]
    moved = _run(seq, E, R, W=int(rng.integers(1, 6)), moves=int(rng.integers(1, 3)),
                 spare=int(rng.integers(1, 4)))
    assert moved > 0  # long tails trigger at least one rebalance


@pytest.mark.parametrize("seed", range(4))
def test_cleanup_matches_oracle_on_long_tail_sequences(seed):
    """Step 4 interleaved with the planner: the same reclaimed copies and
    slots, then the same loads, moves and tables (holes and empty home
    slots included)."""
    rng = np.random.default_rng(100 + seed)
    E, R = [(64, 8), (16, 4), (256, 8), (32, 2)][seed]
    hot = rng.choice(E, max(1, int(0.3 * E)), replace=False)
    p = np.ones(E)
    p[hot] = rng.uniform(2, 8)
    p[: E // R] *= 2.0
    p /= p.sum()
    seq = [rng.multinomial(int(rng.integers(100, 5000)), p) for _ in range(40)]
    moved = _run(seq, E, R, W=int(rng.integers(1, 4)), moves=int(rng.integers(1, 3)),
                 spare=int(rng.integers(1, 3)), cleanup_every=int(rng.integers(2, 5)))
    assert moved > 0


def test_cleanup_validation_and_capacity():
    cfg, st, o = _pair(8, 2, 1, 1, 1)
    c = np.array([10, 1, 1, 1, 1, 1, 1, 1], np.int32)
    moe.moe_eplb_observe(st, c)
    assert moe.moe_eplb_rebalance(st, 1) == [(0, 1)]
    L = moe.lib()
    import ctypes
    n = ctypes.c_int32()
    assert L.moe_eplb_cleanup(st.ctypes.data, 0, ctypes.byref(n), None) == 0  # count only
    assert n.value == 1
    assert L.moe_eplb_cleanup(st.ctypes.data, 0, ctypes.byref(n), None) == 0
    assert n.value == 0                                                    # already reclaimed
    assert L.moe_eplb_cleanup(st.ctypes.data, 1, ctypes.byref(n), None) != 0  # no output array
    assert L.moe_eplb_cleanup(None, 0, ctypes.byref(n), None) != 0


def test_planner_matches_oracle_on_worked_and_edge_cases():
    counts = [10] * 16
    counts[5] = 100
    assert _run([counts], 16, 4, 1, 2, 1) == 2
    assert _run([[30, 30, 20, 20]], 4, 2, 1, 2, 1) == 0           # ratio exactly 1.2
    assert _run([[0] * 8] * 3, 8, 2, 2, 2, 1) == 0                 # no traffic
    assert _run([[50, 40, 1, 1, 1, 1, 1, 1]] * 2, 8, 2, 1, 2, 1) == 1
    rng = np.random.default_rng(9)
    seq = [rng.integers(0, 1000, 64) for _ in range(20)]
    _run(seq, 64, 8, 3, 2, 0)                                       # no spare slots


def test_config_validation():
    bad = [dict(n_experts=10, n_ranks=4), dict(n_ranks=0), dict(window=0),
           dict(threshold=0.5), dict(spare_slots=-1), dict(n_ranks=128, n_experts=256)]
    for kw in bad:
        d = dict(n_experts=16, n_ranks=4, window=2, max_moves=2, spare_slots=1, threshold=1.2)
        d.update(kw)
        cfg = moe.make_eplb_config(**d)
        assert moe.moe_eplb_state_bytes(cfg) == 0
    cfg = moe.make_eplb_config(n_experts=16, n_ranks=4, window=2)
    small = np.zeros(8, np.uint8)
    with pytest.raises(moe.MoEError):
        moe.moe_eplb_init(cfg, small)
    st = np.zeros(moe.moe_eplb_state_bytes(cfg), np.uint8)
    moe.moe_eplb_init(cfg, st)
    with pytest.raises(moe.MoEError):
        moe.moe_eplb_observe(st, np.full(16, -1, np.int32))  # negative count
