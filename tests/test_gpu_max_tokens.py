"""Dispatch (EP blog section 2.2, Step 2) at the largest batch the C ABI
accepts, T = 2^20 tokens, through moe_dispatch with index outputs only,
bit-exact against the oracle's stable counting sort.

At this size the (chunk, slot) table is far past the one-block-per-chunk
placement's limit, so the rank, single-block scan and per-pair index
kernels run on 16,384 chunks: a 32-slot rank share (8 M pairs, 7/8 of them
remote) and the 1024-slot, top-16 maximum (16 M pairs; one scan thread per
slot walks every chunk).  Row indices reach 2^24 - 1.

Expert ids: token t takes (a_t + k b_t) mod E for k < K, with a_t uniform and
b_t a uniform odd stride (E a power of two, so the K ids are distinct);
generating them by sorting random keys would need T x E keys.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("expert_router_gemm_amd")

T_MAX = 1 << 20

CASES = [
    # E, K, ep_size, ep_rank
    (256, 8, 8, 5),
    (1024, 16, 1, 0),
]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _expert_ids(T, E, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, E, size=(T, 1), dtype=np.int64)
    b = 2 * rng.integers(0, E // 2, size=(T, 1), dtype=np.int64) + 1
    return ((a + np.arange(K, dtype=np.int64)[None, :] * b) % E).astype(np.int32)


@pytest.mark.parametrize("E,K,ep,rank", CASES)
def test_dispatch_at_maximum_tokens(E, K, ep, rank):
    T = T_MAX
    topk = _expert_ids(T, E, K, seed=E + K)
    assert all(len(set(r)) == K for r in topk[:: T // 64])
    rep_off, rep_slot, slot_experts = oracle.placement(E, ep, rank)
    S = len(slot_experts)
    seed = 11
    counts_r, offsets_r, perm_r, inv_r = oracle.dispatch(
        oracle.slot_map(topk, rep_off, rep_slot, seed), S)

    H = 128  # hidden and inter must be multiples of 128
    shape = moe.make_shape(hidden=H, inter=128, n_experts=E, top_k=K, n_slots=S)
    ws_bytes = moe.moe_workspace_bytes(shape, T)
    assert ws_bytes > 0
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    h = torch.zeros((T, H), dtype=torch.float16, device="cuda")
    ro, rs, tk = d(rep_off), d(rep_slot), d(topk)
    sm = moe.make_slot_map(ro, rs, seed)
    counts = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((S + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    print(f"[max tokens] T={T} E={E} K={K} S={S} chunks={T // 64} ws={ws_bytes >> 20} MiB",
          flush=True)
    moe.moe_dispatch(shape, T, h, tk, sm, None, None, counts, offsets, perm, inv, ws)
    torch.cuda.synchronize()

    P = int(offsets_r[S])
    assert np.array_equal(counts.cpu().numpy(), counts_r)
    assert np.array_equal(offsets.cpu().numpy(), offsets_r)
    assert np.array_equal(inv.cpu().numpy(), inv_r)
    perm_g = perm.cpu().numpy()
    assert np.array_equal(perm_g[:P], perm_r)
    assert np.all(perm_g[P:] == -7), "perm_src written past the dispatched rows"
