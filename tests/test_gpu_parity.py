"""Parity of the HIP path (through libmoe's C ABI) with the CPU oracle.

Bars:
  * bit-exact: routing indices (tokens whose sorted top-(K+1) logits have a
    gap < 1e-5 are excluded and counted), per-slot counts, offsets, the
    dispatch permutation and inverse, copied rows, fp8 codes and scales;
  * |gpu - ref| <= 2e-3 + 2e-2 |ref| elementwise on layer outputs;
  * intermediates with tolerances derived from the arithmetic (see each test).
Stage tests feed the oracle the GPU's own upstream results, so each stage is
judged on identical inputs.  Small dims keep the oracle to seconds while
spanning several tiles and a ragged tail; the full-size cases compare
sampled tokens.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle

pytestmark = pytest.mark.gpu

gh = pytest.importorskip("gpu_harness")

# Workloads at dims the oracle runs in seconds (routing structure unchanged).
SMALL = {
    1: dict(),
    2: dict(T=256, H=1024, I=512),
    3: dict(T=128, H=512, I=256),
    4: dict(T=2048, H=512, I=256),
    5: dict(T=512, H=1024, I=512),
}


def small_cfg(n, seed=None):
    c = moe_synth.config(n, seed=seed)
    kw = SMALL[n]
    if kw:
        c = moe_synth.scaled_config(n, seed=seed, **kw)
    return c


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _check_routing(L, st, tokens=None):
    """Three checks:
      1. GPU logits within the deterministic fp32-accumulation bound of the
         fp64 oracle logits;
      2. the oracle's softmax/top-K run on the GPU's own logits reproduces
         the GPU's indices on every token (same inputs, same fp32 values:
         exact) and its gates to fp32 rounding;
      3. against the oracle's own logits, indices match on every token that
         is not a near tie (sorted top-(K+1) gap < 1e-5); near ties counted.
    Returns the near-tie mask."""
    cfg = L.cfg
    sel = (lambda a: a) if tokens is None else (lambda a: a[tokens])  # noqa: E731
    h = sel(L.h)
    ref_lg = oracle.router_logits(h, L.wr[: cfg.E], L.bias)
    g_lg, g_idx, g_w = sel(st["logits"]), sel(st["topk_idx"]), sel(st["topk_w"])
    bound = gh.logit_error_bound(L, tokens)
    err = np.abs(g_lg.astype(np.float64) - ref_lg)
    assert np.all(err <= bound), f"logit error {err.max():.3e} above bound"
    idx2, w2 = oracle.softmax_topk(g_lg, cfg.K, groups=cfg.groups)
    assert np.array_equal(g_idx, idx2), "top-K kernel differs from the oracle on the same logits"
    assert np.allclose(g_w, w2, rtol=4e-6, atol=1e-9), "gates differ on the same logits"
    ref_idx, _ = oracle.softmax_topk(ref_lg, cfg.K, groups=cfg.groups)
    tie = oracle.near_tie_tokens(ref_lg, cfg.K)
    if cfg.groups:
        # near ties among the group scores decide the kept groups, and
        # near ties inside the kept groups decide the experts
        G, M = cfg.groups
        gmax = ref_lg.reshape(len(ref_lg), G, -1).max(2)
        tie = tie | oracle.near_tie_tokens(gmax, M)
        order = np.lexsort((np.broadcast_to(np.arange(G), gmax.shape), -gmax), axis=1)
        kept = np.zeros_like(gmax, dtype=bool)
        np.put_along_axis(kept, order[:, :M], True, axis=1)
        masked = np.where(np.repeat(kept, ref_lg.shape[1] // G, axis=1), ref_lg, -1e30)
        tie = tie | oracle.near_tie_tokens(masked, cfg.K)
    ok = ~tie
    assert np.array_equal(g_idx[ok], ref_idx[ok]), "top-k differs on a non-near-tie token"
    if cfg.n_shared:
        z = (h.astype(np.float64) @ L.wr[cfg.E].astype(np.float64))
        ref_gs = 1.0 / (1.0 + np.exp(-z))
        assert np.allclose(sel(st["shared_gate"]), ref_gs, rtol=1e-5, atol=1e-6)
    print(f"[routing] tokens={len(ref_lg)} near_ties={int(tie.sum())} "
          f"max|dlogit|={err.max():.2e}")
    return tie


def _check_dispatch(L, st):
    cfg = L.cfg
    S = len(L.slot_experts)
    # the oracle builds its own table and is fed the GPU's top-k
    rep = moe_synth.replica_expert(cfg)
    ro, rs, _ = oracle.placement(cfg.E, cfg.ep_size, L.rank, replica_of=rep)
    slot = oracle.slot_map(st["topk_idx"], ro, rs, L.seed)
    counts, offsets, perm, inv = oracle.dispatch(slot, S)
    assert np.array_equal(st["counts"], counts)
    assert np.array_equal(st["offsets"], offsets)
    assert np.array_equal(st["perm_src"], perm)
    assert np.array_equal(st["inv_pos"], inv)
    assert np.all(st["perm_tail"] == -7), "rows past P must stay untouched"
    toks = perm // cfg.K
    if cfg.dispatch == "fp8":
        q, s = oracle.quant_e4m3_rows(L.h[toks]) if len(toks) else (np.zeros((0, cfg.H), np.uint8), np.zeros(0, np.float32))
        assert np.array_equal(st["x_perm"], q), "fp8 codes differ"
        assert np.array_equal(st["x_scale"], s), "fp8 scales differ"
    else:
        assert np.array_equal(st["x_perm"], L.h[toks]), "dispatched rows differ"
    return slot


def _check_ffn(L, st):
    """y rows against the oracle SwiGLU on the GPU's own dispatched rows.
    Tolerance: the output bar (fp16 y).  Gathering the rows from h through
    perm_src must give bit-identical hm."""
    cfg = L.cfg
    off = st["offsets"]
    if st["hm_gather"] is not None:
        assert np.array_equal(st["hm_gather"].view(np.uint8), st["hm"].view(np.uint8))
    dec = oracle.e4m3_decode_table()
    for s in range(len(L.slot_experts)):
        a, b = off[s], off[s + 1]
        if a == b:
            continue
        if cfg.dispatch == "fp8":
            x = dec[st["x_perm"][a:b]].astype(np.float32) * st["x_scale"][a:b, None]
        else:
            x = st["x_perm"][a:b]
        y, hm = oracle.expert_rows(x.astype(np.float64), *L.expert(L.slot_experts[s]), want_hm=True)
        gh.assert_close(st["hm"][a:b], hm, f"hm slot {s}")
        gh.assert_close(st["y"][a:b], y, f"y slot {s}")
    if cfg.n_shared:
        for j in range(cfg.n_shared):
            y = oracle.expert_rows(L.h.astype(np.float64), *[m[j] for m in L.shared])
            gh.assert_close(st["shared_y"][j * L.T:(j + 1) * L.T], y, f"shared expert {j}")


def _check_combine(L, st):
    cfg = L.cfg
    shy = None
    if cfg.n_shared:
        shy = st["shared_y"].astype(np.float32).reshape(cfg.n_shared, L.T, cfg.H)
    ref = oracle.combine(st["y"].astype(np.float32), st["inv_pos"], st["topk_w"], shy,
                         st["shared_gate"])
    gh.assert_close(st["out"], ref, "combine")
    none_local = np.all(st["inv_pos"] < 0, axis=1)
    if not cfg.n_shared:
        assert np.all(st["out"][none_local] == 0), "rows with no local pair must be exact zeros"


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("seed_off", [0, 100, 200])
def test_stages_and_layer_small(n, seed_off):
    cfg = small_cfg(n, seed=moe_synth.config(n).seed + seed_off)
    print(f"[case] workload {n} {cfg}", flush=True)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    _check_dispatch(L, st)
    _check_ffn(L, st)
    _check_combine(L, st)
    # the fused entry point runs the same kernels: bitwise equal
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8))
    # end to end against the oracle's own routing (near-tie tokens excluded)
    ref = gh.oracle_forward(L)
    assert np.array_equal(ref["topk_idx"][~tie], st["topk_idx"][~tie])
    err = gh.assert_close(out, ref["out"], "layer output", rows=~tie)
    print(f"[layer] workload {n} P={st['P']} max|d|={err:.3e} near_ties={int(tie.sum())}")


def test_layer_is_deterministic():
    cfg = small_cfg(5)
    L = gh.build_layer(cfg)
    a = gh.gpu_forward(L).cpu().numpy()
    b = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("T", [0, 1, 63, 65, 130])
def test_ragged_and_empty_batches(T):
    cfg = moe_synth.scaled_config(2, T=T, H=256, I=128, seed=21)
    L = gh.build_layer(cfg)
    if T == 0:
        out = torch.empty((0, cfg.H), dtype=torch.float16, device=gh.DEV)
        ws = gh.ws_for(L, 0)
        import expert_router_gemm_amd as moe
        moe.moe_layer_forward(L.shape, L.wmap, L.smap, 0, L.d["h"], out, ws)
        torch.cuda.synchronize()
        return
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    _check_dispatch(L, st)
    ref = gh.oracle_forward(L)
    gh.assert_close(st["out"], ref["out"], "layer", rows=~tie)


def test_hot_expert_spans_several_row_blocks():
    """One expert takes every token (a group of T > 64 rows: several 64-row
    blocks and the 4-tile path), most others get none."""
    cfg = moe_synth.scaled_config(2, T=200, H=256, I=128, seed=22)
    bias = np.zeros(cfg.E, np.float32)
    bias[[3, 17]] = 50.0  # experts 3 and 17 (both local on rank 0) win every token
    L = gh.build_layer(cfg, bias_override=bias)
    st = gh.gpu_stages(L)
    _check_routing(L, st)
    _check_dispatch(L, st)
    assert st["counts"][3] == cfg.T and st["counts"][17] == cfg.T
    _check_ffn(L, st)
    ref = gh.oracle_forward(L)
    gh.assert_close(st["out"], ref["out"], "layer")


def test_no_local_pair_gives_exact_zeros():
    cfg = moe_synth.scaled_config(2, T=70, H=256, I=128, seed=23)
    bias = np.zeros(cfg.E, np.float32)
    bias[100:108] = 50.0  # every token picks experts 100..107 (rank 3)
    L = gh.build_layer(cfg, bias_override=bias)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.all(out.view(np.uint16) == 0)


def test_rank_shares_sum_to_full_layer():
    """EP simulation on one GPU: the 8 rank shares' partial outputs add up to
    the full layer's routed output; every (t, k) is local on one rank."""
    base = moe_synth.scaled_config(2, T=96, H=256, I=128, seed=24)
    full_cfg = moe_synth.scaled_config(2, T=96, H=256, I=128, seed=24, ep_size=1)
    full = gh.gpu_forward(gh.build_layer(full_cfg)).cpu().numpy().astype(np.float64)
    tot = np.zeros_like(full)
    seen = None
    for r in range(8):
        L = gh.build_layer(base, rank=r)
        st = gh.gpu_stages(L)
        tot += st["out"].astype(np.float64)
        m = (st["inv_pos"] >= 0).astype(int)
        seen = m if seen is None else seen + m
    assert np.all(seen == 1)
    gh.assert_close(tot, full, "sum of rank shares", atol=4e-3)


def test_dead_replica_sends_traffic_to_survivor():
    """Section 6.3 replica table with the remote copy removed: every pair of
    the replicated expert is computed on the local replica slot."""
    import expert_router_gemm_amd as moe
    cfg = small_cfg(5)
    L = gh.build_layer(cfg)
    rep = moe_synth.replica_expert(cfg)
    off2, slot2 = moe.drop_replica(L.rep_off, L.rep_slot, rep, 0)
    L.d["rep_off"], L.d["rep_slot"] = gh.to_dev(off2), gh.to_dev(slot2)
    L.smap = moe.make_slot_map(L.d["rep_off"], L.d["rep_slot"], L.seed)
    st = gh.gpu_stages(L)
    n_rep = int((st["topk_idx"] == rep).sum())
    assert st["counts"][len(L.slot_experts) - 1] == n_rep
    ro, rs, _ = oracle.placement(cfg.E, cfg.ep_size, 0, replica_of=rep)
    lo = ro[rep]
    rs2 = np.delete(rs, lo)
    ro2 = ro.copy()
    ro2[rep + 1:] -= 1
    slot = oracle.slot_map(st["topk_idx"], ro2, rs2, L.seed)
    c, o, p, i = oracle.dispatch(slot, len(L.slot_experts))
    assert np.array_equal(st["counts"], c) and np.array_equal(st["perm_src"], p)


def test_fp8_codes_exhaustive_over_fp16_magnitudes():
    """Dispatch quantises with per-row scale 448/amax: sweep rows built from
    every positive finite fp16 value (with signs) and compare codes and
    scales with the oracle's codec bit for bit."""
    import expert_router_gemm_amd as moe
    vals = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)  # all positive finite
    H = 512
    n = (len(vals) + H - 1) // H
    x = np.zeros(n * H, np.float16)
    x[: len(vals)] = vals
    rng = np.random.default_rng(5)
    x = (x * np.where(rng.random(x.size) < 0.5, -1, 1).astype(np.float16)).reshape(n, H)
    x = x[rng.permutation(n)]
    T, K = n, 1
    shape = moe.make_shape(hidden=H, inter=128, n_experts=1, top_k=1, n_slots=1,
                           dispatch=moe.MOE_FP8_E4M3)
    h = gh.to_dev(x)
    idx = torch.zeros((T, K), dtype=torch.int32, device=gh.DEV)
    rep_off = gh.to_dev(np.array([0, 1], np.int32))
    rep_slot = gh.to_dev(np.array([0], np.int32))
    sm = moe.make_slot_map(rep_off, rep_slot, 0)
    xp = torch.empty((T, H), dtype=torch.uint8, device=gh.DEV)
    xs = torch.empty((T,), dtype=torch.float32, device=gh.DEV)
    counts = torch.empty(1, dtype=torch.int32, device=gh.DEV)
    offs = torch.empty(2, dtype=torch.int32, device=gh.DEV)
    perm = torch.empty(T, dtype=torch.int32, device=gh.DEV)
    inv = torch.empty((T, K), dtype=torch.int32, device=gh.DEV)
    ws = torch.empty(moe.moe_workspace_bytes(shape, T), dtype=torch.uint8, device=gh.DEV)
    moe.moe_dispatch(shape, T, h, idx, sm, xp, xs, counts, offs, perm, inv, ws)
    torch.cuda.synchronize()
    q, s = oracle.quant_e4m3_rows(x)
    assert np.array_equal(xs.cpu().numpy(), s)
    assert np.array_equal(xp.cpu().numpy(), q)


def test_dense_topk_equals_experts():
    """top_k = E = S: every token uses every expert (dense softmax MoE)."""
    cfg = moe_synth.scaled_config(1, T=40, H=256, I=128, E=8, K=8, n_shared=0, seed=25)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    assert np.all(st["counts"] == cfg.T)
    ref = gh.oracle_forward(L)
    gh.assert_close(st["out"], ref["out"], "dense layer", atol=1e-5, rtol=1e-4)


def test_maximum_experts_top_k_slots_and_shared():
    """The largest shapes the ABI accepts for routing and placement: E = S =
    1024 (identity map), top_k = 16, 16 shared experts, at tiny dense dims:
    the 16-wide top-K path, the general dispatch (S > 256) and 16 secondary
    groups in the expert launches."""
    cfg = moe_synth.scaled_config(3, T=48, H=128, I=128, E=1024, K=16, n_shared=16,
                                  long_tail=False, seed=61)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    _check_dispatch(L, st)
    assert int(st["counts"].sum()) == cfg.T * cfg.K
    ref = gh.oracle_forward(L)
    gh.assert_close(st["out"], ref["out"], "layer output", rows=~tie)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8))


@pytest.mark.parametrize("T", [70, 40000])
def test_single_expert_is_a_plain_swiglu_ffn(T):
    """E = K = S = 1: every token's gate is softmax over one logit = 1, so
    the layer is the textbook SwiGLU FFN y = W_d (SiLU(W_g h) * W_u h),
    checked against torch on the CPU in float64.  T = 70 runs the weight
    stream; T = 40000 the tiled router (one valid logit column) and tiled
    expert GEMMs on one group of 157 row tiles, split over the XCDs."""
    cfg = moe_synth.scaled_config(2, T=T, H=256, I=128, E=1, K=1, ep_size=1, seed=62)
    L = gh.build_layer(cfg)
    out = gh.gpu_forward(L).cpu().numpy().astype(np.float64)
    g, u, d = (torch.from_numpy(m.astype(np.float64)) for m in L.expert(0))
    h = torch.from_numpy(L.h.astype(np.float64))
    ref = (torch.nn.functional.silu(h @ g.T) * (h @ u.T)) @ d.T
    gh.assert_close(out, ref.numpy(), "single-expert layer")


@pytest.mark.parametrize("T,H,E,K,n_shared,groups", [
    (500, 128, 256, 12, 1, (2, 1)),
    (33, 256, 8, 5, 1, None),
    (64, 256, 16, 13, 2, None),
])
def test_layer_equals_staged_when_shared_and_routed_sizes_differ(T, H, E, K, n_shared, groups):
    """Decode-sized full layers whose routed groups expect 12 or more rows
    and whose shared experts, estimated as n_shared * T / E rows, fewer:
    the two sides of the size at which the down projection's weight stream
    changes shape (inter 512, where the two shapes sum K in different
    orders).  The layer must equal the staged calls bit for bit (it runs
    the shared experts in their own launches here instead of inside the
    routed ones) and the oracle within the bar."""
    kw = dict(n_groups=groups[0], topk_groups=groups[1]) if groups else {}
    cfg = moe_synth.scaled_config(3, T=T, H=H, I=512, E=E, K=K, n_shared=n_shared, ep_size=1,
                                  long_tail=False, seed=64 + T, **kw)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8)), "layer != staged"
    ref = gh.oracle_forward(L)
    gh.assert_close(out, ref["out"], "layer output", rows=~tie)


@pytest.mark.parametrize("groups", [None, (10, 3)])
def test_expert_count_not_a_multiple_of_the_wave(groups):
    """E = 100 (lanes past E hold no expert in the top-K kernel), K = 5, full
    layer resident, with and without a group limit."""
    kw = dict(n_groups=groups[0], topk_groups=groups[1]) if groups else {}
    cfg = moe_synth.scaled_config(2, T=96, H=256, I=128, E=100, K=5, ep_size=1, seed=63, **kw)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    _check_dispatch(L, st)
    ref = gh.oracle_forward(L)
    gh.assert_close(st["out"], ref["out"], "layer output", rows=~tie)


# ------------------------------------------------------------ full sizes


FULL_SAMPLE = {2: 32, 3: 12, 4: 24, 5: 32}
TILE_ROWS = 256  # row tile of the LDS-tiled expert GEMMs


def _strata_rows(offsets, rng, tile=TILE_ROWS):
    """Rows that cover every (slot, row tile): the first and last row of
    each tile of each non-empty slot, plus one drawn at random."""
    rows = []
    for s in range(len(offsets) - 1):
        a, b = int(offsets[s]), int(offsets[s + 1])
        for t0 in range(a, b, tile):
            t1 = min(b, t0 + tile)
            rows += [t0, t1 - 1, int(rng.integers(t0, t1))]
    return np.unique(np.asarray(rows, np.int64))


def _check_ffn_rows(L, st, rows):
    """hm and y of the given dispatched rows against the oracle's SwiGLU on
    the GPU's own dispatched inputs (fp8: its codes and scales), expert by
    expert (regenerated one at a time, not kept).  Returns max |d| of y."""
    cfg = L.cfg
    off = st["offsets"]
    slot_of_row = np.searchsorted(off, rows, side="right") - 1
    dec = oracle.e4m3_decode_table() if cfg.dispatch == "fp8" else None
    need = sorted(set(int(s) for s in slot_of_row))
    worst = 0.0
    for e, w in moe_synth.iter_experts(cfg, [int(L.slot_experts[s]) for s in need]):
        for s in [s for s in need if int(L.slot_experts[s]) == e]:
            r = rows[slot_of_row == s]
            if cfg.dispatch == "fp8":
                x = dec[st["x_perm"][r]].astype(np.float32) * st["x_scale"][r, None]
            else:
                x = L.h[st["perm_src"][r] // cfg.K]
            y, hm = oracle.expert_rows(x.astype(np.float64), *w, want_hm=True)
            gh.assert_close(st["hm"][r], hm, f"hm slot {s} rows {r.min()}..{r.max()}")
            worst = max(worst, gh.assert_close(st["y"][r], y, f"y slot {s}"))
    return worst


@pytest.mark.slow
@pytest.mark.parametrize("n,groups", [(2, None), (5, None), (4, None), (3, None), (2, (8, 4))])
def test_full_size_sampled(n, groups):
    """Full workload sizes in the launch configuration the benchmark times
    (with --groups G,M for the group-limited case):
      * routing of a token sample and the whole dispatch exactly;
      * the expert GEMMs (hm and y, every feature) on rows of every
        (slot, 256-row tile): the full-length K loops and workgroups that
        chain several items, element by element;
      * layer outputs on the token sample within the output bar."""
    cfg = moe_synth.config(n)
    if groups:
        cfg = moe_synth.config(n, n_groups=groups[0], topk_groups=groups[1])
    print(f"[case] full workload {n} {cfg.name} groups={groups}", flush=True)
    L = gh.build_layer(cfg, keep_host_weights=False)
    st = gh.gpu_stages(L)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8))
    rng = np.random.default_rng(n)
    tok = np.sort(rng.choice(cfg.T, FULL_SAMPLE[n], replace=False))
    tie = _check_routing(L, st, tokens=tok)
    _check_dispatch(L, st)
    rows = _strata_rows(st["offsets"], rng)
    if st["hm_gather"] is not None:  # rows gathered from h give the same hm
        assert np.array_equal(st["hm_gather"].view(np.uint8), st["hm"].view(np.uint8))
    dy = _check_ffn_rows(L, st, rows)
    for j in range(cfg.n_shared):  # shared experts: every token is a row
        t = _strata_rows(np.array([0, cfg.T]), rng, tile=64)
        y = oracle.expert_rows(L.h[t].astype(np.float64), *[m[j] for m in L.shared])
        gh.assert_close(st["shared_y"][j * cfg.T + t], y, f"shared expert {j}")
    L.experts.clear()
    ref = gh.oracle_forward(L, tokens=tok)
    err = gh.assert_close(out[tok], ref["out"], "layer output (sample)", rows=~tie)
    print(f"[full] workload {n} P={st['P']} ffn rows={len(rows)} (max |dy| {dy:.3e}) "
          f"sample={len(tok)} max|d|={err:.3e}")


@pytest.mark.slow
def test_layer_at_maximum_tokens():
    """T = 2^20 tokens (the C ABI's limit) with the rank-share routing of the
    decode workload (32 local slots of 256 experts, top-8) and H = I = 128:
    the tiled router, top-K over a million tokens, dispatch through the
    single-block scan, groups of ~32 K rows in the tiled expert GEMMs and a
    million-block combine (and the same combine in the down projection's
    tail, MOE_F_FUSED_COMBINE, bitwise equal).  Routing of a sample and the whole dispatch
    exact, layer outputs on the sample within the output bar."""
    cfg = moe_synth.scaled_config(2, T=1 << 20, H=128, I=128, seed=64)
    print(f"[case] maximum tokens T={cfg.T} H={cfg.H} I={cfg.I}", flush=True)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8))
    # the combine in the down projection's tail: thousands of completed
    # (token, tile)s per workgroup, many rounds of tokens with no local pair
    fused = gh.gpu_forward(L, fused_combine=True).cpu().numpy()
    assert np.array_equal(fused.view(np.uint8), out.view(np.uint8))
    tok = np.sort(np.random.default_rng(64).choice(cfg.T, 64, replace=False))
    tie = _check_routing(L, st, tokens=tok)
    _check_dispatch(L, st)
    ref = gh.oracle_forward(L, tokens=tok)
    err = gh.assert_close(out[tok], ref["out"], "layer output (sample)", rows=~tie)
    print(f"[max tokens] P={st['P']} sample={len(tok)} max|d|={err:.3e}")


def test_prefill_tiled_path_small():
    """T = 4096 rank share: the router (T >= 2048, K split in 2 slices) and
    the routed FFN (>= 64 expected rows per group) take the LDS-tiled kernel."""
    cfg = moe_synth.scaled_config(4, T=4096, H=256, I=128, seed=31)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    _check_dispatch(L, st)
    _check_ffn(L, st)
    _check_combine(L, st)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8))
    ref = gh.oracle_forward(L)
    err = gh.assert_close(out, ref["out"], "layer output", rows=~tie)
    print(f"[tiled] P={st['P']} max|d|={err:.3e} near_ties={int(tie.sum())}")


@pytest.mark.parametrize("T,H,I", [(3000, 640, 384), (8192, 1024, 512)])
def test_tiled_feature_tiles_and_ragged_rows(T, H, I):
    """Prefill-sized groups on the LDS-tiled kernel over several feature
    tiles (gate/up: 128 features per tile, I = 384 three tiles; down: 256
    per tile, H = 640 two and a half), ragged row tails, K = H and K = I
    both several 64-wide steps, items spread over the XCDs in contiguous
    eighths; every stage and the layer against the oracle."""
    cfg = moe_synth.scaled_config(4, T=T, H=H, I=I, seed=34)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    _check_dispatch(L, st)
    _check_ffn(L, st)
    _check_combine(L, st)
    ref = gh.oracle_forward(L)
    err = gh.assert_close(st["out"], ref["out"], "layer output", rows=~tie)
    # the layer with the combine in the tiled down projection's tail
    out = gh.gpu_forward(L, fused_combine=True).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8))
    print(f"[tiled] T={T} H={H} I={I} P={st['P']} max|d|={err:.3e}")


def test_tiled_shared_and_ragged_groups():
    """fp16 16-expert layer with a shared expert at T = 1000: routed groups
    (~125 rows) and the shared group (1000 rows, not a multiple of 128) on
    the tiled kernel, full layer, against the oracle."""
    cfg = moe_synth.scaled_config(1, T=1000, H=256, I=128, dtype="f16", seed=32)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    _check_dispatch(L, st)
    _check_ffn(L, st)
    _check_combine(L, st)
    ref = gh.oracle_forward(L)
    gh.assert_close(st["out"], ref["out"], "layer output", rows=~tie)
    # combine in the routed down projection's tail (shared rows first)
    out = gh.gpu_forward(L, fused_combine=True).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8))


@pytest.mark.parametrize("H", [1536, 7168])
def test_tiled_router_k_split_with_shared_gate(H):
    """Router on the tiled kernel with the shared-gate column (N = E + 1, a
    ragged feature tile) and a ragged token tail (T = 2100): 34 tiles, so
    H = 1536 splits K in 6 slices of 4 K steps and H = 7168 in 8 slices of
    14 (the split closest to 256 workgroups); routing is checked token by
    token."""
    cfg = moe_synth.scaled_config(1, T=2100, H=H, I=128, dtype="f16", seed=33)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    print(f"[tiled router] H={H} near_ties={int(tie.sum())}")


@pytest.mark.parametrize("n,G,M", [(2, 8, 4), (3, 8, 2), (5, 16, 3), (1, 4, 2)])
def test_group_limited_routing(n, G, M):
    """Group-limited routing (M of G contiguous expert groups by their best
    logit): the stages and the layer against the oracle, and every token's
    experts inside at most M groups."""
    cfg = small_cfg(n)
    cfg = moe_synth.scaled_config(n, T=cfg.T, H=cfg.H, I=cfg.I, n_groups=G, topk_groups=M)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    tie = _check_routing(L, st)
    gsz = cfg.E // G
    assert all(len(set((row // gsz).tolist())) <= M for row in st["topk_idx"])
    _check_dispatch(L, st)
    ref = gh.oracle_forward(L)
    gh.assert_close(st["out"], ref["out"], "layer output", rows=~tie)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8))
    print(f"[groups {G}/{M}] workload {n} near_ties={int(tie.sum())}")


def test_profiled_entry_matches_and_records_stage_events():
    import expert_router_gemm_amd as moe
    cfg = small_cfg(3)
    L = gh.build_layer(cfg)
    ref = gh.gpu_forward(L).cpu().numpy()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    out = torch.empty((L.T, cfg.H), dtype=torch.float16, device=gh.DEV)
    ws = gh.ws_for(L)
    moe.moe_layer_forward_profiled(L.shape, L.wmap, L.smap, L.T, L.d["h"], out, ws,
                                   moe.make_profile(ev))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint8), ref.view(np.uint8))
    gaps = [ev[i].elapsed_time(ev[i + 1]) for i in range(5)]
    assert all(g >= 0 for g in gaps) and sum(gaps) > 0
