"""moe_layer_forward_noalloc (the layer with the library's own static
device workspace, for callers that cannot allocate) against
moe_layer_forward with a caller workspace, through the C ABI.  Same kernels
in the same order, so the outputs must be bitwise equal; two calls in a
row, the second with a smaller batch (the array keeps the first call's
contents), then the full-size decode workloads.  Shapes whose workspace
exceeds the array are refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import expert_router_gemm_amd as moe
import moe_synth

pytestmark = pytest.mark.gpu

gh = pytest.importorskip("gpu_harness")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _both(L, T):
    """Outputs of the two entry points on the first T tokens of L."""
    h = L.d["h"][:T].contiguous()
    ref = torch.empty((T, L.cfg.H), dtype=h.dtype, device=gh.DEV)
    ws = torch.empty(moe.moe_workspace_bytes(L.shape, T), dtype=torch.uint8, device=gh.DEV)
    moe.moe_layer_forward(L.shape, L.wmap, L.smap, T, h, ref, ws)
    out = torch.full((T, L.cfg.H), float("nan"), dtype=h.dtype, device=gh.DEV)
    moe.moe_layer_forward_noalloc(L.shape, L.wmap, L.smap, T, h, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.parametrize("n", [1, 2, 3, 5])
def test_noalloc_matches_layer_forward_twice(n):
    """Small dims of each decode-shaped workload: T tokens, then fewer."""
    base = moe_synth.config(n)
    cfg = base if n == 1 else moe_synth.scaled_config(n, T=base.T, H=512, I=256)
    print(f"[case] noalloc workload {n} {cfg}", flush=True)
    L = gh.build_layer(cfg)
    for T in (cfg.T, cfg.T // 2 - 3):
        out, ref = _both(L, T)
        assert np.array_equal(out.view(np.uint8), ref.view(np.uint8)), f"T={T}"


@pytest.mark.parametrize("n", [2, 3])
def test_noalloc_full_size_decode(n):
    """The decode workloads at full size (EP=8 rank share T = 256; whole
    layer T = 128 with 2 shared experts), then a smaller batch."""
    cfg = moe_synth.config(n)
    print(f"[case] noalloc full workload {n} {cfg.name}", flush=True)
    L = gh.build_layer(cfg, keep_host_weights=False)
    assert moe.moe_workspace_bytes(L.shape, cfg.T) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    for T in (cfg.T, 37):
        out, ref = _both(L, T)
        assert np.array_equal(out.view(np.uint8), ref.view(np.uint8)), f"T={T}"


def test_noalloc_refuses_a_workspace_beyond_the_array():
    """The rank-share decode workload at T = 1024 needs 146 MiB of
    workspace: refused with MOE_ERR_WORKSPACE before anything is enqueued;
    the output is untouched.  (Its inputs are real, so even a launch would
    only compute the layer.)"""
    cfg = moe_synth.scaled_config(2, T=1024, H=7168, I=2048)
    print(f"[case] noalloc refusal {cfg.name} T={cfg.T}", flush=True)
    L = gh.build_layer(cfg, keep_host_weights=False)
    assert moe.moe_workspace_bytes(L.shape, cfg.T) > moe.MOE_NOALLOC_SCRATCH_BYTES
    out = torch.full((cfg.T, cfg.H), 7.0, dtype=torch.float16, device=gh.DEV)
    st = moe.lib().moe_layer_forward_noalloc(
        ctypes.byref(L.shape), ctypes.byref(L.wmap), ctypes.byref(L.smap), cfg.T,
        L.d["h"].data_ptr(), out.data_ptr(), None)
    torch.cuda.synchronize()
    assert moe.status_str(st) == "MOE_ERR_WORKSPACE"
    assert bool((out == 7.0).all())
