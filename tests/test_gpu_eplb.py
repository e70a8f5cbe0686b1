"""EPLB-lite on the GPU (expert-parallelism blog page, sections 6.2-6.3).

* moe_expert_counts (device histogram, the monitor's input) equals the
  per-expert count of the routing indices, exactly;
* the double-buffered table swap: forwards through table A; the monitor
  and planner add a copy of the hottest expert to this rank's spare slot;
  the copy's weights are written, table B is uploaded to the second buffer
  and the next forward through B matches the oracle run with placement B;
  a forward through table A still gives the old output bit for bit.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from oracle.eplb import EplbOracle

pytestmark = pytest.mark.gpu

gh = pytest.importorskip("gpu_harness")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("T,E,K", [(0, 256, 8), (1, 256, 8), (257, 256, 8), (16384, 256, 8),
                                   (64, 16, 2), (1000, 1000, 16)])
def test_expert_counts_exact(T, E, K):
    import expert_router_gemm_amd as moe
    rng = np.random.default_rng(T + E)
    idx = rng.integers(0, E, (T, K)).astype(np.int32)
    if T > 1:
        idx[0, 0] = -1          # ids outside [0, E) are not counted
        idx[1, K - 1] = E
    shape = moe.make_shape(hidden=128, inter=128, n_experts=E, top_k=K, n_slots=1)
    counts = torch.full((E,), 77, dtype=torch.int32, device=gh.DEV)  # overwritten
    moe.moe_expert_counts(shape, T, gh.to_dev(idx) if T else counts, counts)
    torch.cuda.synchronize()
    ref = np.bincount(idx[(idx >= 0) & (idx < E)].ravel(), minlength=E)[:E]
    assert np.array_equal(counts.cpu().numpy(), ref)


def test_double_buffered_table_swap_matches_oracle():
    import expert_router_gemm_amd as moe
    cfg = moe_synth.scaled_config(2, T=256, H=512, I=256, seed=41)
    E, R, rank, K = cfg.E, cfg.ep_size, 0, cfg.K
    per = E // R
    # rank 3's experts run hot, rank 0's cold: the planner's target is rank 0
    bias = np.zeros(E, np.float32)
    bias[3 * per: 4 * per] = 1.5
    bias[:per] = -1.0
    h = moe_synth.gen_hidden(cfg)
    wr = moe_synth.gen_router(cfg)
    spare = 1
    S = per + spare
    ecfg = moe.make_eplb_config(n_experts=E, n_ranks=R, window=1, max_moves=1,
                                spare_slots=spare)
    st = np.zeros(moe.moe_eplb_state_bytes(ecfg), np.uint8)
    moe.moe_eplb_init(ecfg, st)
    offA, slotA, seA = moe.moe_eplb_slot_map(st, ecfg, rank)
    assert list(seA) == list(range(per))

    # expert weights in the fragment layout: each slot packed as it is loaded
    pk = lambda a: moe.pack_weights(torch.from_numpy(a).to(gh.DEV))  # noqa: E731
    G = torch.zeros((S, cfg.I, cfg.H), dtype=torch.float16, device=gh.DEV)
    U = torch.zeros_like(G)
    D = torch.zeros((S, cfg.H, cfg.I), dtype=torch.float16, device=gh.DEV)
    host = {}
    for s, (e, (g, u, d)) in enumerate(moe_synth.iter_experts(cfg, seA)):
        G[s].copy_(pk(g)), U[s].copy_(pk(u))
        D[s].copy_(pk(d))
        host[int(e)] = (g, u, d)
    shape = moe.make_shape(hidden=cfg.H, inter=cfg.I, n_experts=E, top_k=K, n_slots=S,
                           w_layout=moe.MOE_W_FRAG)
    hd, wrd, bd = gh.to_dev(h), gh.to_dev(wr), gh.to_dev(bias)
    w = moe.make_weights(w_router=wrd, bias=bd, w_gate=G, w_up=U, w_down=D)
    # two device tables (the double buffer), sized for the largest table
    nnz_max = E + R * spare
    tab = [(torch.zeros(E + 1, dtype=torch.int32, device=gh.DEV),
            torch.zeros(nnz_max, dtype=torch.int32, device=gh.DEV)) for _ in range(2)]
    tab[0][0].copy_(torch.from_numpy(offA))
    tab[0][1][: len(slotA)].copy_(torch.from_numpy(slotA))
    mapA = moe.make_slot_map(tab[0][0], tab[0][1], cfg.seed)
    ws = torch.empty(moe.moe_workspace_bytes(shape, cfg.T), dtype=torch.uint8, device=gh.DEV)
    outA = torch.empty((cfg.T, cfg.H), dtype=torch.float16, device=gh.DEV)
    moe.moe_layer_forward(shape, w, mapA, cfg.T, hd, outA, ws)

    # monitor: route once more to read this forward's per-expert counts
    idx = torch.empty((cfg.T, K), dtype=torch.int32, device=gh.DEV)
    tw = torch.empty((cfg.T, K), dtype=torch.float32, device=gh.DEV)
    moe.moe_route(shape, cfg.T, hd, wrd, bd, idx, tw, None, None, ws)
    counts = torch.empty(E, dtype=torch.int32, device=gh.DEV)
    moe.moe_expert_counts(shape, cfg.T, idx, counts)
    c = counts.cpu().numpy()
    assert int(c.sum()) == cfg.T * K
    moe.moe_eplb_observe(st, c)
    o = EplbOracle(E, R, window=1, max_moves=1, spare_slots=spare)
    o.observe(c)
    _, imb = moe.moe_eplb_loads(st, R)
    assert imb > 1.2
    moves = moe.moe_eplb_rebalance(st, 1)
    assert moves == o.rebalance()
    assert len(moves) == 1 and moves[0][1] == rank and 3 * per <= moves[0][0] < 4 * per
    e_new = moves[0][0]
    offB, slotB, seB = moe.moe_eplb_slot_map(st, ecfg, rank)
    assert list(seB) == list(range(per)) + [e_new]

    # the copy's weights first, then table B into the other buffer
    g, u, d = moe_synth.gen_expert(cfg, e_new)
    host[e_new] = (g, u, d)
    G[per].copy_(pk(g)), U[per].copy_(pk(u))
    D[per].copy_(pk(d))
    tab[1][0].copy_(torch.from_numpy(offB))
    tab[1][1][: len(slotB)].copy_(torch.from_numpy(slotB))
    mapB = moe.make_slot_map(tab[1][0], tab[1][1], cfg.seed)
    outB = torch.empty_like(outA)
    moe.moe_layer_forward(shape, w, mapB, cfg.T, hd, outB, ws)
    outA2 = torch.empty_like(outA)
    moe.moe_layer_forward(shape, w, mapA, cfg.T, hd, outA2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(outA2.cpu().numpy().view(np.uint16), outA.cpu().numpy().view(np.uint16))

    lg = oracle.router_logits(h, wr, bias)
    tie = oracle.near_tie_tokens(lg, K)
    ref = oracle.layer_forward(h=h, w_router=wr, bias=bias, w_sg=None,
                               slot_weights=[host[int(e)] for e in seB], shared=None,
                               rep_off=offB, rep_slot=slotB, seed=cfg.seed, K=K,
                               fp8_dispatch=False)
    gh.assert_close(outB.cpu().numpy(), ref["out"], "layer output (table B)", rows=~tie)
    # the new copy took part of the hot expert's traffic on this rank
    slots = oracle.slot_map(ref["topk_idx"], offB, slotB, cfg.seed)
    assert (slots == per).sum() > 0
    print(f"[eplb] move {moves} imbalance {imb:.3f} pairs on the copy {(slots == per).sum()}")

    # step 4: once table A's work has drained, cleanup reclaims the copy the
    # migration was taken from (rank 3's home copy of e_new); rank 0's table
    # C then sends every pair of e_new to its copy here
    rec = moe.moe_eplb_cleanup(st, ecfg)
    assert rec == o.cleanup() == [(e_new, 3, e_new - 3 * per)]
    offC, slotC, seC = moe.moe_eplb_slot_map(st, ecfg, rank)
    assert list(seC) == list(seB)  # rank 0's slots unchanged
    assert list(slotC[offC[e_new]:offC[e_new + 1]]) == [per]
    tab[0][0].copy_(torch.from_numpy(offC))
    tab[0][1].zero_()
    tab[0][1][: len(slotC)].copy_(torch.from_numpy(slotC))
    mapC = moe.make_slot_map(tab[0][0], tab[0][1], cfg.seed)
    outC = torch.empty_like(outA)
    moe.moe_layer_forward(shape, w, mapC, cfg.T, hd, outC, ws)
    torch.cuda.synchronize()
    refC = oracle.layer_forward(h=h, w_router=wr, bias=bias, w_sg=None,
                                slot_weights=[host[int(e)] for e in seC], shared=None,
                                rep_off=offC, rep_slot=slotC, seed=cfg.seed, K=K,
                                fp8_dispatch=False)
    gh.assert_close(outC.cpu().numpy(), refC["out"], "layer output (table C)", rows=~tie)
    slotsC = oracle.slot_map(refC["topk_idx"], offC, slotC, cfg.seed)
    assert (slotsC == per).sum() == (refC["topk_idx"] == e_new).sum()
    print(f"[eplb] cleanup {rec}: all {(slotsC == per).sum()} pairs of expert {e_new} on the copy")
