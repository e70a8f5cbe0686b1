"""The fragment weight layout MOE_W_FRAG (include/moe.h).

* CPU: this file's numpy packer puts every byte where the header's formula
  says (byte 256q + 16r + c of fragment (i, j) is byte 64j + 16q + c of row
  16i + r).
* GPU: moe_pack_weights is exactly that permutation (bitwise, fp16 and fp32,
  one and several matrices, past the kernel's grid-stride size), and every
  entry point gives bitwise the same results on packed weights as on the
  row-major ones: the same 16-byte operand pieces reach the same lanes in the
  same order, so not a rounding changes.  Checked on every small workload
  through the staged calls and the fused layer, and at full size in the
  launch configuration the benchmark times (decode on the weight-stream
  kernel, prefill on the LDS-tiled kernel).  The row-major path is therefore
  pinned to the oracle by the parity tests, which run on packed weights.
"""
import ctypes

import numpy as np
import pytest
import torch

import moe_synth

moe = pytest.importorskip("expert_router_gemm_amd")


def np_pack(w: np.ndarray) -> np.ndarray:
    """[..., rows, cols] row-major -> the same array in the fragment layout."""
    rows, cols = w.shape[-2], w.shape[-1]
    lead = w.shape[:-2]
    b = np.ascontiguousarray(w).view(np.uint8).reshape(*lead, rows, -1)
    rb = b.shape[-1]
    assert rows % 16 == 0 and rb % 64 == 0
    x = b.reshape(*lead, rows // 16, 16, rb // 64, 4, 16)  # (i, r, j, q, c)
    n = len(lead)
    x = x.transpose(*range(n), n, n + 2, n + 3, n + 1, n + 4)  # (i, j, q, r, c)
    return np.ascontiguousarray(x).reshape(*lead, rows, rb).view(w.dtype).reshape(w.shape)


def test_numpy_packer_follows_the_header_formula():
    rng = np.random.default_rng(7)
    for rows, cols, dt in ((32, 64, np.float16), (16, 48, np.float32), (48, 96, np.float16)):
        w = rng.standard_normal((rows, cols)).astype(dt)
        src = w.view(np.uint8).reshape(rows, -1)
        dst = np_pack(w).view(np.uint8).reshape(-1)
        rb = src.shape[1]
        for n in range(rows):
            for bb in range(rb):
                i, r, j, q, c = n // 16, n % 16, bb // 64, (bb % 64) // 16, bb % 16
                off = (i * (rb // 64) + j) * 1024 + 256 * q + 16 * r + c
                assert dst[off] == src[n, bb]
    # a whole fragment is one operand tile: lane 16q + r holds row r, K quarter q
    w = np.arange(16 * 32, dtype=np.float16).reshape(16, 32)
    frag = np_pack(w).reshape(64, 8)
    for lane in range(64):
        q, r = lane // 16, lane % 16
        assert np.array_equal(frag[lane], w[r, 8 * q:8 * q + 8])


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return "cuda:0"


@pytest.mark.gpu
@pytest.mark.parametrize("dt,shape", [
    (torch.float16, (1, 16, 32)), (torch.float16, (3, 64, 128)), (torch.float32, (2, 32, 48)),
    (torch.float32, (1, 16, 16)), (torch.float16, (2, 2048, 7168)),  # 3.7M units: grid-stride
])
def test_pack_is_the_header_permutation(dt, shape):
    dev = _gpu()
    print(f"[case] pack {dt} {shape}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(11)
    bits = torch.randint(-32768, 32767, shape, dtype=torch.int16, generator=g)
    w = bits.view(torch.float16) if dt == torch.float16 else \
        torch.randn(shape, generator=g, dtype=torch.float32)
    got = moe.pack_weights(w.to(dev))
    torch.cuda.synchronize()
    want = np_pack(w.numpy())
    assert np.array_equal(got.cpu().numpy().view(np.uint8), want.view(np.uint8))


@pytest.mark.gpu
def test_pack_of_no_matrix_enqueues_nothing():
    dev = _gpu()
    a = torch.ones((16, 32), dtype=torch.float16, device=dev)
    b = torch.zeros_like(a)
    moe.moe_pack_weights(moe.MOE_F16, 0, 16, 32, a, b)
    torch.cuda.synchronize()
    assert int(b.count_nonzero()) == 0
    with pytest.raises(moe.MoEError):  # in place: src and dst overlap
        moe.moe_pack_weights(moe.MOE_F16, 1, 16, 32, a, a)


def _same(a, b, what):
    if a is None and b is None:
        return
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, what
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{what} differs between layouts"


@pytest.mark.gpu
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_layouts_bitwise_equal_small(n):
    _gpu()
    import gpu_harness as gh
    from test_gpu_parity import small_cfg
    cfg = small_cfg(n)
    print(f"[case] layouts, workload {n} {cfg}", flush=True)
    res = {}
    for lay in (moe.MOE_W_ROWMAJOR, moe.MOE_W_FRAG):
        L = gh.build_layer(cfg, w_layout=lay, keep_host_weights=False)
        assert L.shape.w_layout == lay
        st = gh.gpu_stages(L)
        st["fused"] = gh.gpu_forward(L).cpu().numpy()
        res[lay] = st
        del L
    a, b = res[moe.MOE_W_ROWMAJOR], res[moe.MOE_W_FRAG]
    for k in ("hm", "hm_gather", "y", "shared_y", "out", "fused", "topk_idx", "offsets"):
        _same(a[k], b[k], k)


def _packed_twin(L):
    """The layer's weights packed into new tensors, and its shape with
    w_layout = MOE_W_FRAG (the row-major ones stay in place)."""
    d = {k: moe.pack_weights(L.d[k]) for k in ("G", "U", "D", "SG", "SU", "SD") if k in L.d}
    s = L.shape
    shape = moe.Shape(*[getattr(s, f) for f, _ in s._fields_])
    shape.w_layout = moe.MOE_W_FRAG
    w = moe.make_weights(w_router=L.d["wr"], bias=L.d["bias"], w_gate=d["G"], w_up=d["U"],
                         w_down=d["D"], sh_gate=d.get("SG"), sh_up=d.get("SU"),
                         sh_down=d.get("SD"))
    return shape, w, d


@pytest.mark.gpu
@pytest.mark.slow
@pytest.mark.parametrize("n", [3, 2, 5, 4])
def test_layouts_bitwise_equal_full_size(n):
    """Full-size workloads, the fused layer as the benchmark calls it: decode
    (weight-stream GEMMs; 2, 3, 5) and the 16384-token prefill (LDS-tiled
    GEMMs; 4)."""
    _gpu()
    import gpu_harness as gh
    cfg = moe_synth.config(n)
    print(f"[case] layouts at full size, workload {n} {cfg}", flush=True)
    L = gh.build_layer(cfg, w_layout=moe.MOE_W_ROWMAJOR, keep_host_weights=False)
    ws = gh.ws_for(L)
    out = [torch.empty((L.T, cfg.H), dtype=L.d["h"].dtype, device="cuda:0") for _ in range(2)]
    moe.moe_layer_forward(L.shape, L.wmap, L.smap, L.T, L.d["h"], out[0], ws)
    shape, w, keep = _packed_twin(L)
    moe.moe_layer_forward(shape, w, L.smap, L.T, L.d["h"], out[1], ws)
    torch.cuda.synchronize()
    a, b = (o.cpu().numpy() for o in out)
    assert np.isfinite(a.astype(np.float32)).all()
    _same(a, b, f"layer output, workload {n}")
    del keep


@pytest.mark.gpu
def test_frag_layout_value_is_validated():
    _gpu()
    import gpu_harness as gh
    from test_gpu_parity import small_cfg
    L = gh.build_layer(small_cfg(3), keep_host_weights=False)
    s = L.shape
    bad = moe.Shape(*[getattr(s, f) for f, _ in s._fields_])
    bad.w_layout = 2
    out = torch.empty((L.T, L.cfg.H), dtype=L.d["h"].dtype, device="cuda:0")
    st = moe.lib().moe_layer_forward(ctypes.byref(bad), ctypes.byref(L.wmap), ctypes.byref(L.smap),
                                     L.T, L.d["h"].data_ptr(), out.data_ptr(),
                                     gh.ws_for(L).data_ptr(), 1 << 40, None)
    assert st == 1  # MOE_ERR_INVALID_ARG, nothing enqueued
