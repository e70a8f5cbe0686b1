"""Expert GEMMs on the LDS-tiled kernel at group sizes on the tile edges,
called through libmoe's C ABI (moe_expert_ffn_up, moe_expert_ffn_down) and
compared with the oracle's SwiGLU expert (EP blog section 2.2, Step 3).

Groups of 0, 1, 127, 128, 129, 255, 256, 257, 300 and 513 rows: empty
groups, 256-row tiles whose second row half is empty (those waves skip
their fragment reads and MFMAs), exact tile multiples and one-row tails.
The x rows are read three ways: already permuted, gathered through a row
index (as the gate/up GEMM gathers h through perm_src; direct-to-LDS loads
from per-lane addresses) and shared (every group reads the same rows, as
the shared experts do).  H = 512 (the down projection's output spans two
256-feature tiles), I = 384 (gate/up: three tiles of 128 features).  Both
weight layouts: row-major (XOR-swizzled LDS rows) and the fragment layout
(fragment-ordered LDS).

Bar: |gpu - ref| <= 2e-3 + 2e-2 |ref| on hm and y (fp16 outputs, fp32
accumulation); rows past the last group are never written.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle

pytestmark = pytest.mark.gpu

gh = pytest.importorskip("gpu_harness")
moe = pytest.importorskip("expert_router_gemm_amd")

SIZES = [0, 1, 127, 128, 129, 255, 256, 257, 300, 513]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("layout", ["frag", "rowmajor"])
@pytest.mark.parametrize("x_rows", ["permuted", "gather", "shared"])
def test_tiled_expert_gemms_at_tile_edges(x_rows, layout):
    cfg = moe_synth.scaled_config(4, T=sum(SIZES), H=512, I=384, seed=41)
    G = len(SIZES)
    offsets = np.concatenate([[0], np.cumsum(SIZES)]).astype(np.int32)
    P = int(offsets[-1])
    experts = [moe_synth.gen_expert(cfg, e) for e in range(G)]
    wg = np.stack([e[0] for e in experts])
    wu = np.stack([e[1] for e in experts])
    wd = np.stack([e[2] for e in experts])
    if x_rows == "shared":
        x = moe_synth.gen_hidden(cfg, T=max(SIZES))
        src = np.concatenate([np.arange(n) for n in SIZES]).astype(np.int64)
        gather = None
        mode = moe.MOE_X_SHARED
    elif x_rows == "gather":
        x = moe_synth.gen_hidden(cfg, T=P + 7)
        src = np.random.default_rng(41).permutation(P + 7)[:P].astype(np.int64)
        gather = src.astype(np.int32)  # top_k = 1: x row = gather[r]
        mode = moe.MOE_X_GATHER
    else:
        x = moe_synth.gen_hidden(cfg, T=P)
        src = np.arange(P, dtype=np.int64)
        gather = None
        mode = moe.MOE_X_PERMUTED

    # est. rows per group (cap_rows / n_experts) >= 64 selects the tiled kernel
    frag = layout == "frag"
    shape = moe.make_shape(hidden=cfg.H, inter=cfg.I, n_experts=G, top_k=1, n_slots=G,
                           w_layout=moe.MOE_W_FRAG if frag else moe.MOE_W_ROWMAJOR)
    cap = P + 64  # rows past the last group stay untouched
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    xd, wgd, wud, wdd, offd = d(x), d(wg), d(wu), d(wd), d(offsets)
    if frag:
        wgd, wud, wdd = (moe.pack_weights(t) for t in (wgd, wud, wdd))
    gd = d(gather) if gather is not None else None
    sentinel = torch.tensor(12345.0, dtype=torch.float16)
    hm = torch.full((cap, cfg.I), sentinel.item(), dtype=torch.float16, device="cuda")
    y = torch.full((cap, cfg.H), sentinel.item(), dtype=torch.float16, device="cuda")
    print(f"[tiled edges] x_rows={x_rows} layout={layout} groups={SIZES} P={P}", flush=True)
    moe.moe_expert_ffn_up(shape, G, cap, xd, moe.MOE_F16, None, mode, gd, offd, wgd, wud, hm)
    moe.moe_expert_ffn_down(shape, G, cap, hm, offd, wdd, y)
    torch.cuda.synchronize()
    hm_g, y_g = hm.cpu().numpy(), y.cpu().numpy()

    for g in range(G):
        a, b = offsets[g], offsets[g + 1]
        if a == b:
            continue
        rows = x[src[a:b]].astype(np.float64)
        y_ref, hm_ref = oracle.expert_rows(rows, wg[g], wu[g], wd[g], want_hm=True)
        gh.assert_close(hm_g[a:b], hm_ref, f"hm group {g} ({b - a} rows)")
        gh.assert_close(y_g[a:b], y_ref, f"y group {g} ({b - a} rows)")
    assert np.all(hm_g[P:] == sentinel.numpy()), "hm rows past the groups were written"
    assert np.all(y_g[P:] == sentinel.numpy()), "y rows past the groups were written"


def test_prefill_layer_repeats_bit_for_bit():
    """The direct-to-LDS pipeline has no run-to-run freedom (fixed K order
    per output, explicit load waits): a prefill-sized layer (T = 8192, the
    tiled router, the fused dispatch placement and the 256-row expert tiles
    with ragged groups) gives identical bits on five launches."""
    cfg = moe_synth.scaled_config(4, T=8192, H=1024, I=512, seed=43)
    L = gh.build_layer(cfg)
    first = gh.gpu_forward(L).cpu().numpy()
    for _ in range(4):
        again = gh.gpu_forward(L).cpu().numpy()
        assert np.array_equal(first.view(np.uint8), again.view(np.uint8))


def test_tiled_more_groups_than_threads():
    """1,024 expert slots, the most the tiled kernels take: every workgroup
    builds its prefix of row tiles per group over two chunks of 512 groups
    (one per thread), carrying the first chunk's total into the second.  A
    full 1024-expert top-16 layer with a shared expert at T = 19200 (300
    rows per slot on average, 124-517: one to three row tiles, most with a
    tail), H = I = 128, on the
    tiled router and expert GEMMs: routing on a token sample, the whole
    dispatch, hm and y on rows covering every (slot, row tile), the combine
    on every token, the layer on the sample against the oracle and equal to
    the staged calls, with the combine as its own launch and in the down
    projection's tail."""
    import test_gpu_parity as tp
    cfg = moe_synth.scaled_config(3, T=19200, H=128, I=128, E=1024, K=16, n_shared=1,
                                  long_tail=False, seed=71)
    print(f"[case] tiled, 1024 groups: {cfg}", flush=True)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    c = st["counts"]
    assert len(c) == 1024 and c.min() < 256 < c.max(), "slots of one and of several row tiles"
    rng = np.random.default_rng(cfg.seed)
    tok = np.sort(rng.choice(cfg.T, 48, replace=False))
    tie = tp._check_routing(L, st, tokens=tok)
    tp._check_dispatch(L, st)
    rows = tp._strata_rows(st["offsets"], rng)
    dy = tp._check_ffn_rows(L, st, rows)
    tp._check_combine(L, st)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8)), "layer != staged"
    fused = gh.gpu_forward(L, fused_combine=True).cpu().numpy()
    assert np.array_equal(fused.view(np.uint8), out.view(np.uint8)), "fused combine differs"
    ref = gh.oracle_forward(L, tokens=tok)
    err = gh.assert_close(out[tok], ref["out"], "layer output (sample)", rows=~tie)
    print(f"[tiled, 1024 groups] P={st['P']} rows/slot {int(st['counts'].min())}.."
          f"{int(st['counts'].max())} ffn rows={len(rows)} (max |dy| {dy:.2e}) max|d|={err:.2e}")
