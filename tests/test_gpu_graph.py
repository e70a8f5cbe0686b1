"""The layer under HIP graph capture (the no-allocation entry point's callers).

moe_layer_forward_noalloc and moe_layer_forward enqueue kernel launches only
(no allocation, copy, memset or synchronisation), so a caller can capture
them once and replay the graph.  Each test captures a decode-sized layer,
then replays it several times with the program's own eager work in between
(another forward that rewrites the same static workspace, an in-place change
of the input, host synchronisations) and checks every replay bit for bit
against an eager call on the same input.  The eager path is pinned to the
oracle by the parity tests.
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


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint8)


@pytest.mark.parametrize("entry", ["noalloc", "workspace"])
@pytest.mark.parametrize("n", [2, 3, 5])
def test_captured_layer_replays_match_eager(n, entry):
    from test_gpu_parity import small_cfg
    cfg = small_cfg(n)
    print(f"[case] graph capture, {entry}, workload {n} {cfg}", flush=True)
    L = gh.build_layer(cfg, keep_host_weights=False)
    T, H = L.T, cfg.H
    dev = gh.DEV
    ws = gh.ws_for(L)

    def forward(h, out, stream=None):
        if entry == "noalloc":
            moe.moe_layer_forward_noalloc(L.shape, L.wmap, L.smap, T, h, out, stream)
        else:
            moe.moe_layer_forward(L.shape, L.wmap, L.smap, T, h, out, ws, stream)

    h = L.d["h"]                       # the graph's input buffer
    h0 = h.clone()
    h1 = torch.flip(h0, dims=[0]).contiguous()  # a second input: the tokens reversed
    out = torch.empty((T, H), dtype=h.dtype, device=dev)
    ref = {}
    for name, src in (("h0", h0), ("h1", h1)):
        h.copy_(src)
        e = torch.empty_like(out)
        forward(h, e)  # eager (also sets up the per-device state before capture)
        torch.cuda.synchronize()
        ref[name] = _bits(e)
    assert not np.array_equal(ref["h0"], ref["h1"])

    h.copy_(h0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        forward(h, out, s)  # one eager call on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        forward(h, out)
    torch.cuda.synchronize()

    scratch_out = torch.empty_like(out)
    for i, name in enumerate(["h0", "h0", "h1", "h0", "h1", "h1"]):
        # eager work between replays: another forward on the other input
        # (rewrites the workspace the graph uses), then the graph's input
        other = "h1" if name == "h0" else "h0"
        h.copy_(h1 if other == "h1" else h0)
        forward(h, scratch_out)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(scratch_out), ref[other])
        h.copy_(h0 if name == "h0" else h1)
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), ref[name]), f"replay {i} ({name}) differs from eager"
    print(f"[graph] workload {n} {entry}: 6 replays bitwise equal to eager")
