"""A seeded sweep of small layer shapes against the oracle, both weight
layouts.

Sixteen shapes drawn once from a fixed seed: hidden 128..640 and inter
128..512 (multiples of 128, so 1-5 K tiles of the weight stream and 1-4
gate/up feature tiles; inter 512 is where the down projection's weight
stream can split K over the waves), 1..64 experts, top-k 1..8, full layer or a rank
share of an EP group of 2, 4 or 8 (with or without a replica of a remote
hot expert), shared experts on the full layer, fp32 / fp16, fp8 dispatch,
long-tail bias, and 1..300 tokens.  Each shape runs the staged entry points
and the fused layer on packed weights and is checked stage by stage against
the oracle to the bars of test_gpu_parity (routing indices exact outside
near ties, dispatch exact, expert rows and outputs within
|d| <= 2e-3 + 2e-2 |ref|); the fused layer must equal the staged calls bit
for bit, and the layer on row-major weights must equal the packed one bit
for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_synth

pytestmark = pytest.mark.gpu

gh = pytest.importorskip("gpu_harness")
moe = pytest.importorskip("expert_router_gemm_amd")


def _shapes(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        i = len(out)
        dtype = str(rng.choice(["f16", "f16", "f32"]))
        E = int(rng.choice([1, 4, 8, 16, 32, 64]))
        ep = int(rng.choice([d for d in (1, 2, 4, 8) if E % d == 0]))
        cfg = moe_synth.config(
            2, name=f"sweep{i}", T=int(rng.choice([1, 5, 64, 130, 300])),
            H=128 * int(rng.integers(1, 6)), I=128 * int(rng.integers(1, 5)), E=E,
            K=int(rng.integers(1, min(E, 8) + 1)),
            n_shared=int(rng.choice([0, 1, 2])) if ep == 1 else 0, dtype=dtype,
            dispatch="fp8" if dtype == "f16" and rng.random() < 0.3 else "same",
            ep_size=ep, ep_rank=int(rng.integers(0, ep)),
            replica=bool(ep > 1 and rng.random() < 0.4), long_tail=bool(rng.random() < 0.5),
            seed=300 + i)
        if cfg.replica:
            try:
                moe_synth.replica_expert(cfg)
            except ValueError:  # no hot expert outside this rank's share
                cfg = dataclasses.replace(cfg, replica=False)
        out.append(cfg)
    return out


SHAPES = _shapes()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_shape_sweep_against_oracle(i):
    import test_gpu_parity as tp
    cfg = SHAPES[i]
    print(f"[case] sweep {i}: {cfg}", flush=True)
    L = gh.build_layer(cfg)  # packed weights
    st = gh.gpu_stages(L)
    tie = tp._check_routing(L, st)
    tp._check_dispatch(L, st)
    tp._check_ffn(L, st)
    tp._check_combine(L, st)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8)), "fused != staged"
    ref = gh.oracle_forward(L)
    assert np.array_equal(ref["topk_idx"][~tie], st["topk_idx"][~tie])
    gh.assert_close(out, ref["out"], "layer output", rows=~tie)
    R = gh.build_layer(cfg, w_layout=moe.MOE_W_ROWMAJOR, keep_host_weights=False)
    out_rm = gh.gpu_forward(R).cpu().numpy()
    assert np.array_equal(out_rm.view(np.uint8), out.view(np.uint8)), "layouts differ"
    print(f"[sweep] {i}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} K={cfg.K} ep={cfg.ep_size} "
          f"shared={cfg.n_shared} {cfg.dtype}/{cfg.dispatch} replica={cfg.replica} "
          f"P={st['P']} near_ties={int(tie.sum())}")


def test_sweep_spans_the_intended_shapes():
    """The drawn shapes include the corners the sweep is for."""
    assert any(c.E == 1 for c in SHAPES) or any(c.K == 1 for c in SHAPES)
    assert any(c.ep_size > 1 for c in SHAPES) and any(c.ep_size == 1 for c in SHAPES)
    assert any(c.dtype == "f32" for c in SHAPES) and any(c.dispatch == "fp8" for c in SHAPES)
    assert any(c.n_shared > 0 for c in SHAPES)
    assert any(c.T == 1 for c in SHAPES) and any(c.T >= 130 for c in SHAPES)
