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
