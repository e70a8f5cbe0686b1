"""Plain Python oracle of EPLB-lite (TEST INFRASTRUCTURE ONLY).

Expert-parallelism blog page, section 6.2 (EPLB, load balancing without
stopping) and 6.3 (redundant experts), read for one EP group:

  1. monitor:   a sliding window of per-expert token counts; a rank's load
                is the sum over the experts it holds of their counts
  2. detect:    rebalance when max(rank load) / mean(rank load) exceeds a
                threshold (the page's typical value is 1.2)
  3. migrate:   take the hottest one or two experts of the most loaded rank
                and give each a copy on an idle rank; new tokens may then go
                to either copy (section 6.3: a random replica), the old copy
                stays where it is
  4. cleanup:   optional on the page; not modelled

Readings taken where the page leaves a step open:
  * the window counts forwards, not milliseconds: the last W observed
    per-forward histograms are summed;
  * a token routed to an expert with n copies goes to each copy with
    probability 1/n (the replica hash is uniform), so a copy carries
    count / n of that expert's tokens and a rank's load is the sum of
    count_e / n_e over the copies it holds, accumulated in expert order;
  * "hottest expert of the most loaded rank": the copy on that rank with
    the largest per-copy load (ties: lower expert id) among the experts
    that can still get a copy; the target is the least loaded rank (ties:
    lower rank) that holds no copy of it and has a spare slot left; after
    each added copy the loads are recomputed (greedy);
  * max_moves copies are added per triggered rebalance (the page: 1-2);
  * ranks are numbered by the contiguous placement of section 2.1; expert
    e's home copy is on rank e // (E / R) and is never removed.

Plain loops only; every function states the step it follows.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np


class EplbOracle:
    def __init__(self, n_experts: int, n_ranks: int, window: int, threshold: float = 1.2,
                 max_moves: int = 2, spare_slots: int = 1):
        assert n_experts % n_ranks == 0 and window >= 1
        self.E, self.R, self.W = n_experts, n_ranks, window
        self.threshold, self.max_moves, self.spare = threshold, max_moves, spare_slots
        self.per = n_experts // n_ranks
        self.hist: List[List[int]] = []          # last W per-forward histograms
        # copies[e]: ranks holding expert e, home first, then added copies in order
        self.copies: List[List[int]] = [[e // self.per] for e in range(n_experts)]
        self.added: List[List[int]] = [[] for _ in range(n_ranks)]  # experts added per rank

    # 1. monitor
    def observe(self, counts) -> None:
        counts = [int(c) for c in counts]
        assert len(counts) == self.E
        self.hist.append(counts)
        if len(self.hist) > self.W:
            self.hist.pop(0)

    def window_counts(self) -> List[int]:
        tot = [0] * self.E
        for h in self.hist:
            for e in range(self.E):
                tot[e] += h[e]
        return tot

    def loads(self) -> List[float]:
        c = self.window_counts()
        load = [0.0] * self.R
        for e in range(self.E):
            share = c[e] / len(self.copies[e])
            for r in self.copies[e]:
                load[r] += share
        return load

    # 2. detect
    def imbalance(self) -> float:
        load = self.loads()
        mean = sum(load) / self.R
        return max(load) / mean if mean > 0 else 0.0

    # 3. migrate (greedy, max_moves copies)
    def rebalance(self) -> List[Tuple[int, int]]:
        moves: List[Tuple[int, int]] = []
        if not self.imbalance() > self.threshold:
            return moves
        c = self.window_counts()
        for _ in range(self.max_moves):
            load = self.loads()
            hot = max(range(self.R), key=lambda r: (load[r], -r))
            cands = [e for e in range(self.E) if hot in self.copies[e]]
            cands.sort(key=lambda e: (-(c[e] / len(self.copies[e])), e))
            done = False
            for e in cands:
                targets = [r for r in range(self.R)
                           if r not in self.copies[e] and len(self.added[r]) < self.spare]
                if not targets:
                    continue
                tgt = min(targets, key=lambda r: (load[r], r))
                self.copies[e].append(tgt)
                self.added[tgt].append(e)
                moves.append((e, tgt))
                done = True
                break
            if not done:
                break
        return moves

    # the table one rank's forward reads (section 6.3 replica lists)
    def slot_map(self, rank: int):
        """(rep_off [E+1], rep_slot [nnz], slot_experts [S]) for ``rank``:
        home experts in slots 0..per-1, added copies after them in the
        order they were added; each expert lists its copies home first, a
        copy on another rank as -1."""
        slot_of = {}
        slot_experts = list(range(rank * self.per, (rank + 1) * self.per))
        for e in slot_experts:
            slot_of[e] = e - rank * self.per
        for e in self.added[rank]:
            slot_of[e] = len(slot_experts)
            slot_experts.append(e)
        off, slots = [0], []
        for e in range(self.E):
            for r in self.copies[e]:
                slots.append(slot_of[e] if r == rank else -1)
            off.append(len(slots))
        return (np.array(off, np.int32), np.array(slots, np.int32),
                np.array(slot_experts, np.int32))


def bincount_experts(topk_idx: np.ndarray, n_experts: int) -> np.ndarray:
    """Per-expert token counts of one forward (section 6.2 monitor input)."""
    return np.bincount(np.asarray(topk_idx).ravel(), minlength=n_experts).astype(np.int32)


def simulate(seq, **cfg) -> Optional[list]:
    """Run the monitor over a sequence of histograms, rebalancing after each
    one; returns the list of (forward, moves) for the forwards that moved."""
    o = EplbOracle(**cfg)
    out = []
    for i, counts in enumerate(seq):
        o.observe(counts)
        m = o.rebalance()
        if m:
            out.append((i, m))
    return out
