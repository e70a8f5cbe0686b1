"""Concurrent callers: the entry points may be called from several host
threads (include/moe.h); each call owns its workspace and stream.

Two host threads each run moe_layer_forward repeatedly on their own stream
with their own workspace and input, over the same weights, while the other
runs; a third pair of threads does the same through the staged entry
points.  Every output must equal an eager, single-threaded call on the same
input bit for bit (the eager path is pinned to the oracle by the parity
tests).  The no-allocation entry point shares one array per device, so it is
not called concurrently (documented as racing).
"""
import threading

import numpy as np
import pytest
import torch

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


@pytest.mark.parametrize("n", [2, 4])
def test_two_threads_two_streams_match_eager(n):
    from test_gpu_parity import small_cfg
    cfg = small_cfg(n)
    print(f"[case] concurrency, workload {n} {cfg}", flush=True)
    L = gh.build_layer(cfg, keep_host_weights=False)
    T, H = L.T, cfg.H
    h = [L.d["h"].clone(), torch.flip(L.d["h"], dims=[0]).contiguous()]
    ref = []
    for x in h:
        e = torch.empty((T, H), dtype=x.dtype, device=gh.DEV)
        moe.moe_layer_forward(L.shape, L.wmap, L.smap, T, x, e, gh.ws_for(L))
        torch.cuda.synchronize()
        ref.append(_bits(e))
    assert not np.array_equal(ref[0], ref[1])

    reps = 6
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty((T, H), dtype=h[0].dtype, device=gh.DEV) for _ in range(reps)]
            for _ in range(2)]
    wss = [gh.ws_for(L), gh.ws_for(L)]
    errors = []

    def worker(i):
        try:
            for r in range(reps):
                moe.moe_layer_forward(L.shape, L.wmap, L.smap, T, h[i], outs[i][r], wss[i],
                                      streams[i])
        except Exception as exc:  # reported after join
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for r in range(reps):
            assert np.array_equal(_bits(outs[i][r]), ref[i]), f"thread {i} call {r} differs"

    # the staged entry points from two threads (route + dispatch only: the
    # routing outputs are integers and fp32 gates, compared exactly)
    def staged(i, res):
        s = streams[i]
        ws = wss[i]
        K, E, S = cfg.K, cfg.E, len(L.slot_experts)
        idx = torch.empty((T, K), dtype=torch.int32, device=gh.DEV)
        tw = torch.empty((T, K), dtype=torch.float32, device=gh.DEV)
        sg = torch.empty((T,), dtype=torch.float32, device=gh.DEV) if cfg.n_shared else None
        counts = torch.empty((S,), dtype=torch.int32, device=gh.DEV)
        offsets = torch.empty((S + 1,), dtype=torch.int32, device=gh.DEV)
        perm = torch.empty((T * K,), dtype=torch.int32, device=gh.DEV)
        inv = torch.empty((T, K), dtype=torch.int32, device=gh.DEV)
        fp8 = cfg.dispatch == "fp8"
        xp = torch.empty((T * K, H), dtype=torch.uint8, device=gh.DEV) if fp8 else None
        xs = torch.empty((T * K,), dtype=torch.float32, device=gh.DEV) if fp8 else None
        for _ in range(reps):
            moe.moe_route(L.shape, T, h[i], L.d["wr"], L.d["bias"], idx, tw, sg, None, ws, s)
            moe.moe_dispatch(L.shape, T, h[i], idx, L.smap, xp, xs, counts, offsets, perm, inv,
                             ws, s)
        s.synchronize()
        res[i] = [t.cpu().numpy() for t in (idx, tw, counts, offsets, inv)]

    single = [None, None]
    for i in range(2):
        staged(i, single)
    both = [None, None]
    threads = [threading.Thread(target=staged, args=(i, both)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i in range(2):
        for a, b in zip(single[i], both[i]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    print(f"[concurrency] workload {n}: 2 x {reps} layer calls and staged routing on two "
          f"streams from two threads, bitwise equal to eager")
