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
  4. cleanup:   once every request routed with the old table has been
                served, the copy at each migrated expert's original
                position may be reclaimed (optional on the page, under
                memory pressure): a migration then becomes a move

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
    e's home copy is on rank e // (E / R) in that rank's home slot
    e % (E / R); rebalancing never removes a copy;
  * cleanup runs when the caller says the old table has drained; the
    "original position" of a migration is the copy on the overloaded rank
    it was taken from; each (expert, origin) recorded since the last
    cleanup loses that copy, in expert order then rank order, unless it is
    the expert's last one; a reclaimed home slot stays empty, a reclaimed
    added copy leaves a hole in its rank's spare slots that the next copy
    placed on that rank fills (slot numbers never shift).

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
        # spare slots of each rank in slot order: the expert held, or -1 (a hole)
        self.added: List[List[int]] = [[] for _ in range(n_ranks)]
        self.home_live: List[bool] = [True] * n_experts
        self.pending: List[List[bool]] = [[False] * n_ranks for _ in range(n_experts)]

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
                           if r not in self.copies[e] and self._free_spare(r) >= 0]
                if not targets:
                    continue
                tgt = min(targets, key=lambda r: (load[r], r))
                self.copies[e].append(tgt)
                j = self._free_spare(tgt)
                if j < len(self.added[tgt]):
                    self.added[tgt][j] = e        # fill a hole
                else:
                    self.added[tgt].append(e)
                self.pending[e][hot] = True       # the copy it was taken from
                moves.append((e, tgt))
                done = True
                break
            if not done:
                break
        return moves

    def _free_spare(self, r: int) -> int:
        """Index of the first free spare slot of rank r (a hole, else the
        next unused one), or -1 when all spare_slots hold copies."""
        for j, e in enumerate(self.added[r]):
            if e < 0:
                return j
        return len(self.added[r]) if len(self.added[r]) < self.spare else -1

    # 4. cleanup (the old table has drained)
    def cleanup(self) -> List[Tuple[int, int, int]]:
        """Reclaim the original-position copies of the migrations recorded
        since the last cleanup; returns (expert, rank, slot) per reclaimed
        copy (slot: its local slot on that rank)."""
        out = []
        for e in range(self.E):
            for r in range(self.R):
                if not self.pending[e][r]:
                    continue
                self.pending[e][r] = False
                if r not in self.copies[e] or len(self.copies[e]) < 2:
                    continue
                if r == e // self.per and self.home_live[e]:
                    slot = e - r * self.per
                    self.home_live[e] = False
                else:
                    j = self.added[r].index(e)
                    slot = self.per + j
                    self.added[r][j] = -1
                self.copies[e].remove(r)
                out.append((e, r, slot))
        return out

    # the table one rank's forward reads (section 6.3 replica lists)
    def slot_map(self, rank: int):
        """(rep_off [E+1], rep_slot [nnz], slot_experts [S]) for ``rank``:
        home experts in slots 0..per-1, spare slots after them (-1 in
        slot_experts: a reclaimed slot or hole); each expert lists its
        copies in the order they were created (home first while it lives),
        a copy on another rank as -1."""
        slot_of = {}
        slot_experts = []
        for s in range(self.per):
            e = rank * self.per + s
            slot_experts.append(e if self.home_live[e] else -1)
            if self.home_live[e]:
                slot_of[e] = s
        for j, e in enumerate(self.added[rank]):
            slot_experts.append(e)
            if e >= 0:
                slot_of[e] = self.per + j
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
