"""The C ABI driven from plain C: tests/c_abi_demo.c (built by build() into
tests/_build/c_abi_demo) reads a layer's inputs from files, allocates its
own device buffers, packs the expert weights with moe_pack_weights, runs
moe_layer_forward and moe_layer_forward_noalloc (bitwise equal, checked in
C) and writes the output.  It must equal, bit for bit, the output of the
same layer driven through the Python binding (whose path is pinned to the
oracle by the parity tests).  The program runs as a child process.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import moe_synth

pytestmark = pytest.mark.gpu

gh = pytest.importorskip("gpu_harness")
moe = pytest.importorskip("expert_router_gemm_amd")

DEMO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "c_abi_demo")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("cfg", [
    moe_synth.config(1),  # fp32, 16 experts, top-2, one shared expert
    moe_synth.config(3, T=64, H=256, I=128, E=32, K=4, long_tail=False, seed=33),  # fp16, 2 shared
], ids=["fp32", "fp16"])
def test_c_program_matches_the_binding(cfg, tmp_path):
    assert os.path.exists(DEMO), "tests/_build/c_abi_demo missing: run __graft_entry__.build()"
    print(f"[case] C ABI demo {cfg}", flush=True)
    L = gh.build_layer(cfg)
    assert L.bias is None and cfg.ep_size == 1
    want = gh.gpu_forward(L).cpu().numpy()
    S = len(L.slot_experts)
    dt = cfg.np_dtype
    d = str(tmp_path)
    with open(os.path.join(d, "shape.txt"), "w") as f:
        f.write(f"{cfg.H} {cfg.I} {cfg.E} {cfg.K} {S} {cfg.n_shared} {L.T} "
                f"{gh.act_code(cfg)} {L.seed}\n")
    L.h.astype(dt).tofile(os.path.join(d, "h.bin"))
    L.wr.astype(dt).tofile(os.path.join(d, "wr.bin"))
    for i, name in enumerate(("gate", "up", "down")):
        np.stack([L.expert(e)[i] for e in L.slot_experts]).astype(dt).tofile(
            os.path.join(d, name + ".bin"))
        if cfg.n_shared:
            np.ascontiguousarray(L.shared[i]).astype(dt).tofile(os.path.join(d, f"sh_{name}.bin"))
    L.rep_off.astype(np.int32).tofile(os.path.join(d, "rep_off.bin"))
    L.rep_slot.astype(np.int32).tofile(os.path.join(d, "rep_slot.bin"))
    r = subprocess.run([DEMO, d], capture_output=True, text=True, timeout=120)
    print(r.stdout.strip(), r.stderr.strip())
    assert r.returncode == 0, r.stderr
    got = np.fromfile(os.path.join(d, "out.bin"), dtype=dt).reshape(want.shape)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
