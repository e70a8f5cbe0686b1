"""A seeded sweep of prefill-sized layer shapes on the LDS-tiled kernels,
against the oracle, with the combine as its own launch and in the down
projection's tail.

Six shapes drawn once from a fixed seed: 1,500-6,000 tokens, hidden
256-1,536 and inter 128-768 (multiples of 128, so both GEMMs meet narrower
last feature tiles), 8-64 experts and top-k 2-8 with at least 64 expected
rows per slot (the tiled expert GEMMs; from 2,048 tokens on the tiled
router too), the full layer or a rank share of EP = 2/4/8 (any rank), a
shared expert on some, long-tail routing on some, fp16.  Each shape:
routing on a token sample and the whole dispatch exactly; hm and y on rows
covering every (slot, 256-row tile) against the oracle's SwiGLU; the
combine on every token; the layer equal to the staged calls bit for bit
with and without MOE_F_FUSED_COMBINE; layer outputs on the sample within
the output bar.
"""
import numpy as np
import pytest
import torch

import moe_synth

pytestmark = pytest.mark.gpu

gh = pytest.importorskip("gpu_harness")
moe = pytest.importorskip("expert_router_gemm_amd")


def _shapes(n=6, seed=7070):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        i = len(out)
        E = int(rng.choice([8, 16, 32, 64]))
        ep = int(rng.choice([d for d in (1, 2, 4, 8) if E % d == 0 and E // d >= 2]))
        T = int(rng.choice([1500, 3000, 6000]))
        K = int(rng.integers(2, min(E, 8) + 1))
        if T * K // E < 64:  # the expected rows per slot that pick the tiled GEMMs
            continue
        out.append(moe_synth.config(
            2, name=f"tiled_sweep{i}", T=T, H=128 * int(rng.integers(2, 13)),
            I=128 * int(rng.integers(1, 7)), E=E, K=K, n_shared=int(rng.choice([0, 1])),
            dtype="f16", dispatch="same", ep_size=ep, ep_rank=int(rng.integers(0, ep)),
            replica=False, long_tail=bool(rng.random() < 0.5), seed=700 + i))
    return out


SHAPES = _shapes()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_tiled_shape_against_oracle(i):
    import test_gpu_parity as tp
    cfg = SHAPES[i]
    print(f"[case] tiled sweep {i}: {cfg}", flush=True)
    L = gh.build_layer(cfg)
    st = gh.gpu_stages(L)
    rng = np.random.default_rng(cfg.seed)
    tok = np.sort(rng.choice(cfg.T, 40, replace=False))
    tie = tp._check_routing(L, st, tokens=tok)
    tp._check_dispatch(L, st)
    rows = tp._strata_rows(st["offsets"], rng)
    dy = tp._check_ffn_rows(L, st, rows) if len(rows) else 0.0
    tp._check_combine(L, st)
    out = gh.gpu_forward(L).cpu().numpy()
    assert np.array_equal(out.view(np.uint8), st["out"].view(np.uint8)), "layer != staged"
    fused = gh.gpu_forward(L, fused_combine=True).cpu().numpy()
    assert np.array_equal(fused.view(np.uint8), out.view(np.uint8)), "fused combine differs"
    ref = gh.oracle_forward(L, tokens=tok)
    err = gh.assert_close(out[tok], ref["out"], "layer output (sample)", rows=~tie)
    print(f"[tiled sweep] {i}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} K={cfg.K} "
          f"ep={cfg.ep_size}/{cfg.ep_rank} shared={cfg.n_shared} P={st['P']} "
          f"ffn rows={len(rows)} (max |dy| {dy:.2e}) max|d|={err:.2e}")


def test_tiled_sweep_spans_the_intended_shapes():
    assert all(c.T * c.K // c.E >= 64 for c in SHAPES)
    assert any(c.ep_size > 1 for c in SHAPES) and any(c.ep_size == 1 for c in SHAPES)
    assert any(c.n_shared for c in SHAPES) and any(not c.n_shared for c in SHAPES)
    assert any(c.H % 256 for c in SHAPES), "a narrower last feature tile of the down GEMM"
    assert any(c.T >= 2048 for c in SHAPES), "the tiled router"
