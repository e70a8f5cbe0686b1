"""Host-side expert -> local slot tables for libmoe's moe_slot_map.

Expert-parallelism blog page, section 2.1: an EP group of N GPUs splits the
E routed experts into N contiguous ranges, GPU g holding experts
[g*E/N, (g+1)*E/N); the owner is found by integer division, no lookup table.
Section 6.3: a hot expert may get redundant copies on other GPUs and each
token picks one at random.

Layout produced here (CSR over experts): replicas of expert e are
rep_slot[rep_off[e]:rep_off[e+1]], each a local slot or -1 (remote copy).
An extra replica hosted on this GPU takes the next free local slot; its
expert's list is [home copy, extra slot].
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def contiguous_owner(e: int, n_experts: int, ep_size: int) -> int:
    return e // (n_experts // ep_size)


def build_slot_map(n_experts: int, ep_size: int = 1, ep_rank: int = 0,
                   extra_replicas: Optional[Sequence[int]] = None):
    """Returns (rep_off int32 [E+1], rep_slot int32 [nnz], slot_experts int32 [S]).

    slot_experts[s] is the logical expert whose weights slot s must hold."""
    if n_experts % ep_size:
        raise ValueError("n_experts must be a multiple of ep_size")
    per = n_experts // ep_size
    first = ep_rank * per
    slot_experts = list(range(first, first + per))
    extra = {}
    for e in extra_replicas or ():
        if first <= e < first + per:
            raise ValueError(f"expert {e} is already resident on rank {ep_rank}")
        extra[e] = len(slot_experts)
        slot_experts.append(e)
    off = np.zeros(n_experts + 1, np.int32)
    slots = []
    for e in range(n_experts):
        slots.append(e - first if first <= e < first + per else -1)
        if e in extra:
            slots.append(extra[e])
        off[e + 1] = len(slots)
    return off, np.asarray(slots, np.int32), np.asarray(slot_experts, np.int32)


def drop_replica(rep_off: np.ndarray, rep_slot: np.ndarray, expert: int, which: int):
    """Remove replica ``which`` of ``expert`` (e.g. a failed copy); traffic
    then goes to the survivors."""
    lo = int(rep_off[expert])
    if not 0 <= which < int(rep_off[expert + 1]) - lo:
        raise IndexError("no such replica")
    slot = np.delete(rep_slot, lo + which)
    off = rep_off.copy()
    off[expert + 1:] -= 1
    return off, slot
