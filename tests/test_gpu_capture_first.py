"""A prefill-sized layer captured into a HIP graph when the only earlier
eager call used none of the LDS-tiled kernels.

The tiled GEMMs need per-device set-up (their dynamic LDS limit, the count
of resident workgroups) that is not a stream operation.  The library does
it for every tiled kernel on its first call on a device, whatever that call
launches, so a process that has only run decode-sized (weight-stream)
layers eagerly can capture a prefill-sized one.  The scenario needs a
process in which no tiled kernel has run yet, so it runs in a child
process: eager decode-sized layer, then capture of a 4096-token layer
(tiled router and expert GEMMs), replays checked bit for bit against an
eager call of the same layer made after them.
"""
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
import moe_synth, gpu_harness as gh, expert_router_gemm_amd as moe

def forward(L, ws, out, stream=None):
    moe.moe_layer_forward(L.shape, L.wmap, L.smap, L.T, L.d["h"], out, ws, stream)

torch.cuda.init()
dec = gh.build_layer(moe_synth.scaled_config(2, T=256, H=512, I=256, seed=81),
                     keep_host_weights=False)
pre = gh.build_layer(moe_synth.scaled_config(4, T=4096, H=512, I=256, seed=82),
                     keep_host_weights=False)
assert pre.T * pre.cfg.K // pre.cfg.E >= 64, "the prefill layer must take the tiled GEMMs"
ws_d, ws_p = gh.ws_for(dec), gh.ws_for(pre)
o_d = torch.empty((dec.T, dec.cfg.H), dtype=torch.float16, device=gh.DEV)
forward(dec, ws_d, o_d)  # the only eager call before the capture: weight-stream kernels
torch.cuda.synchronize()
print("[child] eager decode-sized layer done", flush=True)

out = torch.empty((pre.T, pre.cfg.H), dtype=torch.float16, device=gh.DEV)
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):
    forward(pre, ws_p, out)
torch.cuda.synchronize()
print("[child] captured the prefill-sized layer", flush=True)
reps = []
for i in range(3):
    out.fill_(0)
    forward(dec, ws_d, o_d)  # eager work between replays
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps.append(out.cpu().numpy().view(np.uint8).copy())
eager = torch.empty_like(out)
forward(pre, ws_p, eager)
torch.cuda.synchronize()
ref = eager.cpu().numpy().view(np.uint8)
for i, r in enumerate(reps):
    assert np.array_equal(r, ref), f"replay {i} differs from eager"
print("[child] 3 replays bitwise equal to eager", flush=True)
"""


def test_capture_of_tiled_layer_after_decode_only_eager_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] capture-first: child process, decode eager then prefill capture", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", CHILD, ROOT], capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-2000:])
    assert r.returncode == 0, f"child failed ({r.returncode}):\n{r.stderr[-3000:]}"
    assert "3 replays bitwise equal to eager" in r.stdout
