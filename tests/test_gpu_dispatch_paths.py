"""Dispatch (EP blog section 2.2, Step 2) on every large-batch path, through
libmoe's C ABI (moe_dispatch with index outputs only), bit-exact against the
oracle's stable counting sort.

Batches above the decode size rank each 64-token chunk, then either place
the pairs with one block per chunk (slot table of at most 256 slots and
64 K chunk x slot entries) or scan with one block and index per pair.  The
cases sit on both sides of that choice: 256 chunks x 256 slots (exactly
64 K), 257 x 256 (one chunk more), a 33-slot rank share with a replica
(hash-chosen copies) and 1024 slots with top-16.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("expert_router_gemm_amd")

CASES = [
    # T, E, K, ep_size, ep_rank, replica_of
    (16384, 256, 8, 1, 0, None),
    (16448, 256, 8, 1, 0, None),
    (4096, 256, 8, 8, 3, 5),
    (2000, 1024, 16, 1, 0, None),
]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("T,E,K,ep,rank,rep", CASES)
def test_dispatch_large_paths_exact(T, E, K, ep, rank, rep):
    rng = np.random.default_rng(T + E + K)
    topk = np.argsort(rng.random((T, E), dtype=np.float32), axis=1)[:, :K].astype(np.int32)
    rep_off, rep_slot, slot_experts = oracle.placement(E, ep, rank, rep)
    S = len(slot_experts)
    seed = 7
    counts_r, offsets_r, perm_r, inv_r = oracle.dispatch(
        oracle.slot_map(topk, rep_off, rep_slot, seed), S)

    H = 128  # hidden and inter must be multiples of 128
    shape = moe.make_shape(hidden=H, inter=128, n_experts=E, top_k=K, n_slots=S)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    h = torch.zeros((T, H), dtype=torch.float16, device="cuda")
    ro, rs, tk = d(rep_off), d(rep_slot), d(topk)
    sm = moe.make_slot_map(ro, rs, seed)
    counts = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((S + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(shape, T), dtype=torch.uint8, device="cuda")
    print(f"[dispatch paths] T={T} E={E} K={K} S={S} chunks={(T + 63) // 64}", flush=True)
    moe.moe_dispatch(shape, T, h, tk, sm, None, None, counts, offsets, perm, inv, ws)
    torch.cuda.synchronize()

    P = int(offsets_r[S])
    assert np.array_equal(counts.cpu().numpy(), counts_r)
    assert np.array_equal(offsets.cpu().numpy(), offsets_r)
    assert np.array_equal(inv.cpu().numpy(), inv_r)
    perm_g = perm.cpu().numpy()
    assert np.array_equal(perm_g[:P], perm_r)
    assert np.all(perm_g[P:] == -7), "perm_src written past the dispatched rows"


@pytest.mark.parametrize("T", [300, 5000])
def test_dispatch_drops_the_later_pair_of_a_repeated_slot(T):
    """A token's pairs should land in distinct slots; when two meet in one
    (repeated ids in a caller's topk_idx, or a table that lists a slot
    under several experts) only the earlier k is dispatched and the later
    gets inv_pos = -1 (include/moe.h).  Expected: the oracle's counting
    sort of the slot map with exactly those later pairs removed.  T = 300
    takes the single-block path, T = 5000 rank + place."""
    E, K, S, seed = 64, 8, 16, 11
    rng = np.random.default_rng(T)
    topk = np.argsort(rng.random((T, E), dtype=np.float32), axis=1)[:, :K].astype(np.int32)
    rep = rng.random(T) < 0.3  # some tokens repeat one of their ids
    k2 = rng.integers(1, K, T)
    k1 = (k2 * rng.random(T)).astype(int)
    topk[rep, k2[rep]] = topk[rep, k1[rep]]
    # every slot listed under 4 experts (e and e + 16, e + 32, e + 48)
    rep_off = np.arange(E + 1, dtype=np.int32)
    rep_slot = (np.arange(E) % S).astype(np.int32)
    slot = oracle.slot_map(topk, rep_off, rep_slot, seed)
    keep = slot.copy()
    for k in range(1, K):
        seen = (slot[:, :k] == slot[:, k:k + 1]).any(1)
        keep[seen & (slot[:, k] >= 0), k] = -1
    assert (keep != slot).sum() > T // 4, "the case must exercise the rule"
    counts_r, offsets_r, perm_r, inv_r = oracle.dispatch(keep, S)

    H = 128
    shape = moe.make_shape(hidden=H, inter=128, n_experts=E, top_k=K, n_slots=S)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    h = torch.zeros((T, H), dtype=torch.float16, device="cuda")
    ro, rs, tk = d(rep_off), d(rep_slot), d(topk)  # kept alive: the map holds raw pointers
    sm = moe.make_slot_map(ro, rs, seed)
    counts = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((S + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(shape, T), dtype=torch.uint8, device="cuda")
    print(f"[dispatch repeated slots] T={T} dropped={(keep != slot).sum()}", flush=True)
    moe.moe_dispatch(shape, T, h, tk, sm, None, None, counts, offsets, perm, inv, ws)
    torch.cuda.synchronize()
    P = int(offsets_r[S])
    assert np.array_equal(counts.cpu().numpy(), counts_r)
    assert np.array_equal(offsets.cpu().numpy(), offsets_r)
    assert np.array_equal(inv.cpu().numpy(), inv_r)
    perm_g = perm.cpu().numpy()
    assert np.array_equal(perm_g[:P], perm_r)
    assert np.all(perm_g[P:] == -7)
