"""The combine fused into the down projection (MOE_F_FUSED_COMBINE).

With the flag set and the routed down projection on the LDS-tiled kernel
(fp16, groups expected to hold >= 64 rows), moe_layer_forward forms the
layer output in that launch's tail instead of a separate combine launch:
the last
workgroup to write one of a token's rows in a 256-feature tile sums the
token's rows for that tile in k order (tickets seeded by dispatch, agent-
scope release/acquire).  Its arithmetic is the combine kernel's, so the
fused layer must equal the staged calls (route, dispatch, ffn, the
separate moe_combine) bit for bit; the staged outputs are checked against
the oracle.  Cases: a rank share with tokens that have no local pair (exact
zeros), the same with a shared expert (those tokens get the shared term
alone), a narrower last feature tile (hidden 640 = 2.5 tiles), a full
layer with shared experts, and a batch large enough that workgroups sum
completed tiles between item batches as well as at the end.
"""
import numpy as np
import pytest
import torch

import moe_synth

pytestmark = pytest.mark.gpu

gh = pytest.importorskip("gpu_harness")
moe = pytest.importorskip("expert_router_gemm_amd")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


CASES = {
    # EP=8 rank share (32 of 256 experts, top-8): 128 expected rows per group
    "share_H640": dict(n=2, T=4096, H=640, I=256, seed=41),
    "share_shared_H640": dict(n=2, T=4096, H=640, I=256, seed=42, n_shared=1),
    # full 16-expert layer with a shared expert (every token local)
    "full_shared": dict(n=1, T=1000, H=384, I=128, seed=43, dtype="f16"),
    # 16384-token rank share: ~1,000 completed (token, tile)s per workgroup
    "share_T16384": dict(n=4, T=16384, H=1024, I=256, seed=44),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_combine_equals_staged(name):
    import test_gpu_parity as tp
    c = dict(CASES[name])
    n = c.pop("n")
    cfg = moe_synth.scaled_config(n, **c)
    print(f"[case] fused combine {name}: {cfg}", flush=True)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    est = cfg.T * cfg.K // cfg.E
    assert est >= 64, "the routed down projection must take the tiled kernel"
    out = gh.gpu_forward(L, fused_combine=True).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8)), "fused != staged"
    # again: the tickets are reseeded every call
    out2 = gh.gpu_forward(L, fused_combine=True).cpu().numpy()
    assert np.array_equal(out2.view(np.uint8), out.view(np.uint8)), "second call differs"
    # and the default (separate combine launch) gives the same bits
    out3 = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out3.view(np.uint8), out.view(np.uint8)), "flag changes the result"
    tp._check_combine(L, st)  # the staged combine against the oracle's, every token
    none_local = (st["inv_pos"] < 0).all(axis=1)
    if cfg.n_shared == 0:
        assert np.all(out[none_local] == 0), "tokens with no local pair must be exact zeros"
    tok = np.sort(np.random.default_rng(cfg.seed).choice(cfg.T, min(cfg.T, 48), replace=False))
    tie = tp._check_routing(L, st, tokens=tok)
    ref = gh.oracle_forward(L, tokens=tok)
    err = gh.assert_close(out[tok], ref["out"], "layer output (sample)", rows=~tie)
    print(f"[fused combine] {name}: T={cfg.T} H={cfg.H} P={st['P']} "
          f"no-local tokens={int(none_local.sum())} max|d|={err:.3e}")


@pytest.mark.parametrize("entry", ["noalloc", "workspace"])
def test_fused_combine_under_graph_capture(entry):
    """The fused path enqueues kernel launches only (dispatch seeds the
    tickets; no memset): captured once with the flag, through the
    no-allocation entry point and through moe_layer_forward, every replay
    equals an eager call bit for bit, with other eager calls on the same
    workspace between the replays."""
    c = dict(CASES["full_shared"])
    n = c.pop("n")
    cfg = moe_synth.scaled_config(n, **c)
    print(f"[case] fused combine under capture ({entry}): {cfg}", flush=True)
    L = gh.build_layer(cfg, keep_host_weights=False)
    shape = type(L.shape).from_buffer_copy(L.shape)
    shape.flags |= moe.MOE_F_FUSED_COMBINE
    T, H = L.T, cfg.H
    ws = gh.ws_for(L)

    def forward(h, out, stream=None):
        if entry == "noalloc":
            moe.moe_layer_forward_noalloc(shape, L.wmap, L.smap, T, h, out, stream)
        else:
            moe.moe_layer_forward(shape, L.wmap, L.smap, T, h, out, ws, stream)

    h = L.d["h"]
    h0 = h.clone()
    h1 = torch.flip(h0, dims=[0]).contiguous()
    ref = {}
    for name, src in (("h0", h0), ("h1", h1)):
        h.copy_(src)
        e = torch.empty((T, H), dtype=h.dtype, device=gh.DEV)
        forward(h, e)
        torch.cuda.synchronize()
        ref[name] = e.cpu().numpy().view(np.uint8)
    out = torch.empty((T, H), dtype=h.dtype, device=gh.DEV)
    h.copy_(h0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        forward(h, out, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward(h, out)
    torch.cuda.synchronize()
    other = torch.empty_like(out)
    for i, name in enumerate(["h0", "h1", "h1", "h0"]):
        h.copy_(h1 if name == "h0" else h0)
        forward(h, other)  # eager call on the other input: rewrites the workspace
        torch.cuda.synchronize()
        h.copy_(h0 if name == "h0" else h1)
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint8), ref[name]), f"replay {i}"
    print(f"[fused combine] {entry}: 4 replays bitwise equal to eager")
