#!/usr/bin/env python3
"""Benchmark of the MoE-layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

One step = one pass of the whole path over one batch resident in HBM: one
call of moe_layer_forward_profiled (router + top-K, dispatch, gate/up and
down grouped GEMMs with the shared experts, combine) through libmoe's C ABI
on torch's current stream; the call records HIP events around the gate/up
GEMM, which give the roofline record.  The same pass without events, a
per-stage breakdown and the staged entry points are reported beside it.

The default workload is the whole DeepSeek-V3 MoE layer at decode: 128
tokens, hidden 7168, top-8 of 256 routed experts with the long-tail routing
of the EP blog's section 6.1, 2 shared experts, all 256 + 2 experts' SwiGLU
7168x2048 weights resident in fp16 (22.5 GB, section 2.1).  After it, the
same run times the prefill workload (one EP=8 rank's 32 experts, 16384
tokens: the compute-bound regime) and reports it under the "prefill" key
with the MFMA fraction of its gate/up GEMM.

Printed: one JSON line with tokens/s, a roofline record for the dominant
kernel (the gate/up weight stream, timed with HIP events on the stream it
runs on), the layer's HBM fraction counting only the bytes the layer must
move (touched expert weights, shared experts, router, h, out), and the CPU
oracle timed on the host for the same workload (all host threads the run
may use, and one thread).

--summarize-pmc FETCH_DIR WRITE_DIR: turn two `rocprofv3 --pmc FETCH_SIZE`
/ `--pmc WRITE_SIZE` runs of this script (with --copy-calibration) into the
HBM traffic record under profiles/ that later runs report.
"""
from __future__ import annotations

import argparse
import gc
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
DEFAULT_WORKLOAD = 3           # whole layer, decode, T = 128
PREFILL_WORKLOAD = 4           # EP=8 rank share, prefill, T = 16384
# The dominant kernel of a workload: the gate/up weight stream at decode
# sizes, the LDS-tiled gate/up GEMM (256-row tiles, rows gathered) at prefill.
# Its HBM traffic record is keyed by a hash of the sources it is built from.
KERNEL_SOURCES = {
    "stream": ["expert_router_gemm_amd/csrc/gemm_stream.hip",
               "expert_router_gemm_amd/csrc/common.h",
               "expert_router_gemm_amd/csrc/kernels.h"],
    "tiled": ["expert_router_gemm_amd/csrc/gemm_tiled.hip",
              "expert_router_gemm_amd/csrc/common.h",
              "expert_router_gemm_amd/csrc/kernels.h"],
}
DOMINANT = {"stream": "stream_gemm_kernel", "tiled": "tiled_gemm_kernel"}


def dominant_kind(workload: int) -> str:
    return "tiled" if workload == PREFILL_WORKLOAD else "stream"


def kernel_source_hash(kind: str = "stream") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(kind: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{kind}_gemm_swiglu_{workload}.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ setup


LAYOUT_NAME = {"frag": "fragment (MOE_W_FRAG)", "rowmajor": "row-major"}
# where the combine runs (moe_shape.flags)
COMBINE_NAME = {False: "separate launch",
                True: "tail of the tiled down projection where it runs (MOE_F_FUSED_COMBINE)"}


def setup(n: int, keep_host: bool = True, groups=None, w_layout: str = "frag",
          fused_combine: bool = False):
    import numpy as np
    import torch

    import expert_router_gemm_amd as moe
    import moe_synth

    cfg = moe_synth.config(n)
    if groups:
        cfg = moe_synth.config(n, n_groups=groups[0], topk_groups=groups[1])
    dev = "cuda:0"
    rep = moe_synth.replica_expert(cfg)
    rep_off, rep_slot, slot_experts = moe.build_slot_map(cfg.E, cfg.ep_size, cfg.ep_rank,
                                                         [rep] if rep is not None else None)
    S = len(slot_experts)
    tdt = torch.float32 if cfg.dtype == "f32" else torch.float16
    t0 = time.time()
    G = torch.empty((S, cfg.I, cfg.H), dtype=tdt, device=dev)
    U = torch.empty((S, cfg.I, cfg.H), dtype=tdt, device=dev)
    D = torch.empty((S, cfg.H, cfg.I), dtype=tdt, device=dev)
    host_experts = {}
    for s, (e, (g, u, d)) in enumerate(moe_synth.iter_experts(cfg, slot_experts)):
        G[s].copy_(torch.from_numpy(g))
        U[s].copy_(torch.from_numpy(u))
        D[s].copy_(torch.from_numpy(d))
        if keep_host:
            host_experts[e] = (g, u, d)
    h = moe_synth.gen_hidden(cfg)
    wr = moe_synth.gen_router(cfg)
    bias = moe_synth.gen_router_bias(cfg)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa
    d = dict(h=t(h), wr=t(wr), bias=t(bias), G=G, U=U, D=D, ro=t(rep_off), rs=t(rep_slot))
    shared = None
    if cfg.n_shared:
        shared = moe_synth.gen_shared_weights(cfg)
        d.update(SG=t(shared[0]), SU=t(shared[1]), SD=t(shared[2]))
    if w_layout == "frag":
        # expert weights in the fragment layout (moe_pack_weights, once at
        # load time; the row-major copies are freed)
        for k in ("G", "U", "D", "SG", "SU", "SD"):
            if k in d:
                d[k] = moe.pack_weights(d[k])
        G, U, D = d["G"], d["U"], d["D"]
    torch.cuda.synchronize()
    log(f"[bench] generated and uploaded {cfg.name} ({w_layout} expert weights) in "
        f"{time.time() - t0:.1f}s")
    fp8 = cfg.dispatch == "fp8"
    shape = moe.make_shape(hidden=cfg.H, inter=cfg.I, n_experts=cfg.E, top_k=cfg.K, n_slots=S,
                           n_shared=cfg.n_shared,
                           act=moe.MOE_F32 if cfg.dtype == "f32" else moe.MOE_F16,
                           dispatch=moe.MOE_FP8_E4M3 if fp8 else None, shared=cfg.n_shared > 0,
                           n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                           w_layout=moe.MOE_W_FRAG if w_layout == "frag" else moe.MOE_W_ROWMAJOR,
                           fused_combine=fused_combine)
    T, K = cfg.T, cfg.K
    bufs = dict(
        ws=torch.empty(moe.moe_workspace_bytes(shape, T), dtype=torch.uint8, device=dev),
        idx=torch.empty((T, K), dtype=torch.int32, device=dev),
        tw=torch.empty((T, K), dtype=torch.float32, device=dev),
        sg=torch.empty((T,), dtype=torch.float32, device=dev),
        xp=torch.empty((T * K, cfg.H), dtype=torch.uint8 if fp8 else tdt, device=dev),
        xs=torch.empty((T * K,), dtype=torch.float32, device=dev),
        counts=torch.empty((S,), dtype=torch.int32, device=dev),
        offsets=torch.empty((S + 1,), dtype=torch.int32, device=dev),
        perm=torch.empty((T * K,), dtype=torch.int32, device=dev),
        inv=torch.empty((T, K), dtype=torch.int32, device=dev),
        hm=torch.empty((max(T * K, cfg.n_shared * T), cfg.I), dtype=tdt, device=dev),
        y=torch.empty((T * K, cfg.H), dtype=tdt, device=dev),
        shy=torch.empty((max(cfg.n_shared, 1) * T, cfg.H), dtype=tdt, device=dev),
        shoff=t(np.arange(cfg.n_shared + 1, dtype=np.int32) * T),
        out=torch.empty((T, cfg.H), dtype=tdt, device=dev),
        out2=torch.empty((T, cfg.H), dtype=tdt, device=dev),
    )
    wmap = moe.make_weights(w_router=d["wr"], bias=d["bias"], w_gate=G, w_up=U, w_down=D,
                            sh_gate=d.get("SG"), sh_up=d.get("SU"), sh_down=d.get("SD"))
    smap = moe.make_slot_map(d["ro"], d["rs"], cfg.seed)
    return dict(cfg=cfg, shape=shape, d=d, b=bufs, wmap=wmap, smap=smap, S=S, h=h, wr=wr,
                bias=bias, host_experts=host_experts, shared=shared, rep=rep, w_layout=w_layout)


def staged_step(ctx, ev=None):
    """One pass of the hot path through the staged entry points; ev, if
    given, is a list of 6 events recorded at the stage boundaries."""
    import expert_router_gemm_amd as moe
    cfg, shape, d, b = ctx["cfg"], ctx["shape"], ctx["d"], ctx["b"]
    T, S = cfg.T, ctx["S"]
    fp8 = cfg.dispatch == "fp8"
    rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)  # noqa: E731
    rec(0)
    moe.moe_route(shape, T, d["h"], d["wr"], d["bias"], b["idx"], b["tw"],
                  b["sg"] if cfg.n_shared else None, None, b["ws"])
    rec(1)
    # fp8 rows are quantised copies; fp16 rows are gathered by the GEMM
    moe.moe_dispatch(shape, T, d["h"], b["idx"], ctx["smap"], b["xp"] if fp8 else None,
                     b["xs"] if fp8 else None, b["counts"], b["offsets"], b["perm"], b["inv"],
                     b["ws"])
    rec(2)
    if fp8:
        moe.moe_expert_ffn_up(shape, S, T * cfg.K, b["xp"], moe.MOE_FP8_E4M3, b["xs"],
                              moe.MOE_X_PERMUTED, None, b["offsets"], d["G"], d["U"], b["hm"])
    else:
        moe.moe_expert_ffn_up(shape, S, T * cfg.K, d["h"], shape.act, None, moe.MOE_X_GATHER,
                              b["perm"], b["offsets"], d["G"], d["U"], b["hm"])
    rec(3)
    moe.moe_expert_ffn_down(shape, S, T * cfg.K, b["hm"], b["offsets"], d["D"], b["y"])
    rec(4)
    shy = None
    if cfg.n_shared:
        moe.moe_expert_ffn(shape, cfg.n_shared, cfg.n_shared * T, d["h"], shape.act, None,
                           moe.MOE_X_SHARED, None, b["shoff"], d["SG"], d["SU"], d["SD"], b["shy"],
                           b["ws"])
        shy = b["shy"]
    moe.moe_combine(shape, T, b["y"], b["inv"], b["tw"], shy, b["sg"] if cfg.n_shared else None,
                    b["out"])
    rec(5)


def fused_step(ctx):
    import expert_router_gemm_amd as moe
    moe.moe_layer_forward(ctx["shape"], ctx["wmap"], ctx["smap"], ctx["cfg"].T, ctx["d"]["h"],
                          ctx["b"]["out2"], ctx["b"]["ws"])


def profiled_step(ctx, prof):
    import expert_router_gemm_amd as moe
    moe.moe_layer_forward_profiled(ctx["shape"], ctx["wmap"], ctx["smap"], ctx["cfg"].T,
                                   ctx["d"]["h"], ctx["b"]["out2"], ctx["b"]["ws"], prof)


# ------------------------------------------------------------------ accounting


def shared_in_routed_launch(cfg) -> bool:
    """Whether the layer entry runs the shared experts as extra groups of
    the routed gate/up launch: both sides stream weights (fewer than 64
    expected rows per group) and rows are gathered (not fp8 copies)."""
    if not cfg.n_shared or cfg.dispatch == "fp8":
        return False
    return cfg.T * cfg.K // cfg.E < 64 and cfg.n_shared * cfg.T // cfg.E < 64


def algorithmic_work(cfg, counts):
    """Algorithmic bytes and FLOPs of one step, from the routing the step
    produced (per-slot counts; the same input every step).

    layer_bytes: what the layer must move at least -- the weights of every
    touched expert and of the shared experts, the router, h in and out back
    (T*H each).  Intermediates (hm, y) and the softmax/top-K, dispatch and
    combine count as time, not as work.
    up: the gate/up launch of the layer entry -- gate and up weights of the
    touched experts (and of the shared experts when they ride in the same
    launch), each of its input rows read once and its hm rows written once."""
    import numpy as np
    counts = np.asarray(counts)
    P = int(counts.sum())
    touched = int((counts > 0).sum())
    isz = 4 if cfg.dtype == "f32" else 2
    xsz = 1 if cfg.dispatch == "fp8" else isz
    H, I, E, T, K = cfg.H, cfg.I, cfg.E, cfg.T, cfg.K
    n_sh = cfg.n_shared
    merged = shared_in_routed_launch(cfg)
    sh_rows = n_sh * T if merged else 0
    up_groups = touched + (n_sh if merged else 0)
    up = dict(bytes=up_groups * 2 * I * H * isz + (P + sh_rows) * (H * xsz + I * isz)
              + (P * 4 if xsz == 1 else 0),
              flops=2 * 2 * (P + sh_rows) * H * I)
    layer_bytes = ((touched + n_sh) * 3 * H * I * isz + E * H * isz + 2 * T * H * isz)
    layer_flops = (2 * T * H * (E + (n_sh > 0)) + 6 * P * H * I + 6 * n_sh * T * H * I)
    return dict(P=P, touched=touched, up=up, layer_bytes=layer_bytes, layer_flops=layer_flops)


def load_traffic(kind: str, workload: str):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 PMC record, if it was taken on the current kernel source."""
    p = traffic_path(kind, workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    return rec.get("traffic_bytes_per_launch")


# ------------------------------------------------------------------ timing


def time_workload(ctx, K: int, warmup: int, references: bool = True):
    """Warm up, then time K passes of moe_layer_forward_profiled between two
    synchronisations (wall clock).  Every EVERY-th pass records HIP events
    on the launch stream around the gate/up GEMM (events[2], [3]); the
    others pass no events (an event record costs the stream a few µs).
    references: also time the entry point without events, a per-stage
    breakdown and the staged entry points (same kernels)."""
    import torch

    import expert_router_gemm_amd as moe
    for _ in range(warmup):
        fused_step(ctx)
        if references:
            staged_step(ctx)
    torch.cuda.synchronize()
    EVERY = max(1, K // 5)
    ev_up = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for i in range(0, K, EVERY)}
    no_ev = moe.make_profile([])
    profs = [moe.make_profile([None, None, *ev_up[i]]) if i in ev_up else no_ev
             for i in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        profiled_step(ctx, profs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    r = dict(ms_per_step=wall * 1e3 / K,
             up_ms=statistics.mean(a.elapsed_time(b) for a, b in ev_up.values()))
    if not references:
        return r
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        fused_step(ctx)
    e1.record()
    torch.cuda.synchronize()
    r["plain_ms"] = e0.elapsed_time(e1) / K
    ev_all = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for i in range(K):
        profiled_step(ctx, moe.make_profile(ev_all[i]))
    torch.cuda.synchronize()
    names = ["route", "dispatch", "ffn_up", "ffn_down+shared", "combine"]
    r["stage_ms"] = {n: statistics.median(ev[j].elapsed_time(ev[j + 1]) for ev in ev_all)
                     for j, n in enumerate(names)}
    e0.record()
    for _ in range(K):
        staged_step(ctx)
    e1.record()
    torch.cuda.synchronize()
    r["staged_ms"] = e0.elapsed_time(e1) / K
    r["same"] = bool(torch.equal(ctx["b"]["out"], ctx["b"]["out2"]))
    r["step_dist"] = step_distribution(ctx, K)
    return r


def percentiles(v):
    """median, p10 and p90 (nearest rank) of a list of step times."""
    v = sorted(v)

    def rank(q):
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {"median": round(statistics.median(v), 4), "p10": round(rank(0.1), 4),
            "p90": round(rank(0.9), 4), "n": len(v)}


def step_distribution(ctx, K: int):
    """Per-step times of moe_layer_forward: K passes with an event between
    consecutive passes on the launch stream (each record costs the stream a
    few µs, so the mean here sits a little above the timed region's)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ev[0].record()
    for i in range(K):
        fused_step(ctx)
        ev[i + 1].record()
    torch.cuda.synchronize()
    return percentiles([ev[i].elapsed_time(ev[i + 1]) for i in range(K)])


def probe_read_rate(gib: int = 8, reps: int = 5):
    """Best HBM read rate of libmoe_probe.so's slab reader (contiguous 1 KB
    nontemporal wave loads, the decode weight stream's access pattern) over
    a few launch shapes: the measured counterpart of the 8 TB/s peak."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "expert_router_gemm_amd", "libmoe_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.moe_probe_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    nbytes, slab = gib << 30, 1 << 20
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    shapes = [(b, u) for b in (1024, 2048, 4096) for u in (4, 8)]
    out = torch.empty(max(b for b, _ in shapes) * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for blocks, unroll in shapes:
        def launch():
            rc = fn(buf.data_ptr(), nbytes, slab, blocks, unroll, out.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"moe_probe_read returned {rc}")
        launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ms = []
        for _ in range(reps):
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        gbs = nbytes / (min(ms) / 1e3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "blocks": blocks, "unroll": unroll}
    del buf, out
    torch.cuda.empty_cache()
    best.update(bytes=nbytes, slab=slab,
                kernel="libmoe_probe.so read_slabs_kernel (best of blocks 1024/2048/4096 x 4/8 "
                       "1 KB pieces in flight per wave)")
    return best


def reference_rates(reps: int = 20):
    """Measured rates beside the published peaks the fractions use: the
    HBM read probe (probe_read_rate), what the vendor's own kernels reach --
    torch's device copy (read + write) and sum (read only) over 2 GiB of
    fp16, torch.mm on an 8192^3 fp16 product (hipBLASLt).  Context for
    roofline.frac; not part of the layer."""
    import torch
    n = 1 << 30  # fp16 elements: 2 GiB
    x = torch.ones(n, device="cuda:0", dtype=torch.float16)
    y = torch.empty_like(x)
    cp = _timed(lambda: y.copy_(x), 0, reps)
    rd = _timed(lambda: x.sum(dtype=torch.float32), 0, reps)
    del x, y
    torch.cuda.empty_cache()
    nbytes = 2 * n
    hbm = {"copy_gbs": round(2 * nbytes / (cp["us"] / 1e6) / 1e9, 1),
           "read_gbs": round(nbytes / (rd["us"] / 1e6) / 1e9, 1),
           "kernels": "torch copy_ (2 GiB read + 2 GiB written) and sum (2 GiB read), fp16"}
    a = torch.randn(8192, 8192, device="cuda:0", dtype=torch.float16)
    b = torch.randn(8192, 8192, device="cuda:0", dtype=torch.float16)
    mm = _timed(lambda: torch.mm(a, b), 2 * 8192 ** 3, reps)
    del a, b
    torch.cuda.empty_cache()
    return {"hbm": hbm, "hbm_read_probe": probe_read_rate(),
            "mfma": {"tflops": mm["tflops"], "kernel": "torch.mm fp16 8192^3"},
            "published": {"hbm_gbs": HBM_PEAK_GBS, "mfma_f16_tflops": MFMA_F16_PEAK_TFLOPS}}


def kernel_roofline(cfg, work, up_ms, workload_kind):
    """Roofline record of the gate/up launch: algorithmic bytes (decode,
    HBM-bound) or FLOPs (prefill, MFMA-bound) over its live duration."""
    if workload_kind == "stream":
        achieved = work["up"]["bytes"] / (up_ms / 1e3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=load_traffic("stream", cfg.name))
    else:
        achieved = work["up"]["flops"] / (up_ms / 1e3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=MFMA_F16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                    traffic=load_traffic("tiled", cfg.name))
    roof.update(kernel=f"{DOMINANT[workload_kind]} (SwiGLU gate/up, in moe_layer_forward)",
                launch_ms=round(up_ms, 4), algorithmic_bytes=work["up"]["bytes"],
                algorithmic_flops=work["up"]["flops"])
    return roof


def layer_record(work, t):
    ms = t["ms_per_step"]
    gbs = work["layer_bytes"] / (ms / 1e3) / 1e9
    tfs = work["layer_flops"] / (ms / 1e3) / 1e12
    rec = {"entry": "moe_layer_forward_profiled", "hbm_gbs": round(gbs, 1),
           "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "mfma_tflops": round(tfs, 1),
           "mfma_frac": round(tfs / MFMA_F16_PEAK_TFLOPS, 4),
           "algorithmic_bytes": work["layer_bytes"], "algorithmic_flops": work["layer_flops"],
           "rows": work["P"], "touched_slots": work["touched"]}
    if "plain_ms" in t:
        rec.update(no_events_ms=round(t["plain_ms"], 4), staged_calls_ms=round(t["staged_ms"], 4),
                   staged_equals_fused=t["same"],
                   stage_ms={k: round(v, 4) for k, v in t["stage_ms"].items()})
    if "step_dist" in t:
        rec["step_ms"] = t["step_dist"]  # moe_layer_forward, one event per step boundary
    return rec


# ------------------------------------------------------------------ EPLB-lite


def eplb_report(ctx, steps: int = 12):
    """Monitor cost and balance effect of EPLB-lite on this workload's
    routing: the device histogram per forward (HIP events), the host
    observe + rebalance per forward, and the max/mean rank load of the
    simulated EP group (the workload's own, else 8 ranks) after each
    forward's rebalance.  The batch repeats, so the loads settle."""
    import numpy as np
    import torch

    import expert_router_gemm_amd as moe
    cfg, shape, d, b = ctx["cfg"], ctx["shape"], ctx["d"], ctx["b"]
    E, T = cfg.E, cfg.T
    R = cfg.ep_size if cfg.ep_size > 1 else 8
    counts = torch.empty(E, dtype=torch.int32, device="cuda:0")
    moe.moe_route(shape, T, d["h"], d["wr"], d["bias"], b["idx"], b["tw"],
                  b["sg"] if cfg.n_shared else None, None, b["ws"])
    for _ in range(3):
        moe.moe_expert_counts(shape, T, b["idx"], counts)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 50
    e0.record()
    for _ in range(n):
        moe.moe_expert_counts(shape, T, b["idx"], counts)
    e1.record()
    torch.cuda.synchronize()
    counts_us = e0.elapsed_time(e1) * 1e3 / n
    ecfg = moe.make_eplb_config(n_experts=E, n_ranks=R, window=4, max_moves=2, spare_slots=2)
    st = np.zeros(moe.moe_eplb_state_bytes(ecfg), np.uint8)
    moe.moe_eplb_init(ecfg, st)
    host_us, imb, moves = [], [], []
    c = counts.cpu().numpy()
    for _ in range(steps):
        t0 = time.perf_counter()
        moe.moe_eplb_observe(st, c)
        before = moe.moe_eplb_loads(st, R)[1]
        mv = moe.moe_eplb_rebalance(st, 2)
        host_us.append((time.perf_counter() - t0) * 1e6)
        imb.append(round(before, 4))
        moves += mv
    final = moe.moe_eplb_loads(st, R)[1]
    return dict(ranks=R, window=4, max_moves=2, spare_slots=2,
                counts_kernel_us=round(counts_us, 2),
                host_observe_rebalance_us=round(statistics.median(host_us), 1),
                imbalance_per_forward=imb, imbalance_final=round(final, 4),
                moves=[list(m) for m in moves])


# ------------------------------------------------------------------ CPU baseline


def host_threads() -> int:
    """Host threads the run may use: OMP_NUM_THREADS when set (the share
    of the machine this process gets), else the CPU count, at most 16."""
    v = os.environ.get("OMP_NUM_THREADS", "")
    n = int(v) if v.isdigit() and int(v) > 0 else (os.cpu_count() or 1)
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_ram_gb():
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    return round(int(line.split()[1]) / 2 ** 20, 1)
    except OSError:
        pass
    return None


def cpu_baseline(ctx, budget_s: float = 20.0):
    """The oracle (plain C, fp64 accumulation) on the same workload's tokens
    on the host, timed around its layer forward only.  First one thread on
    the first tokens (doubling until about a third of the budget is used),
    then every host thread the run may use, each on its own contiguous
    block of the batch's first tokens (the oracle call releases the
    interpreter lock), sized from the single-thread rate to fill the rest
    of the budget; tokens/s of each."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    cfg = ctx["cfg"]
    ro, rs, se = oracle.placement(cfg.E, cfg.ep_size, cfg.ep_rank, replica_of=ctx["rep"])
    sw = [ctx["host_experts"][int(e)] for e in se]

    def run(tok):
        oracle.layer_forward(h=np.ascontiguousarray(ctx["h"][tok]), w_router=ctx["wr"][: cfg.E],
                             bias=ctx["bias"], w_sg=ctx["wr"][cfg.E] if cfg.n_shared else None,
                             slot_weights=sw, shared=ctx["shared"], rep_off=ro, rep_slot=rs,
                             seed=cfg.seed, K=cfg.K, fp8_dispatch=cfg.dispatch == "fp8",
                             tok_ids=tok, groups=cfg.groups)

    done, t1, n = 0, 0.0, 1
    while done < cfg.T and t1 < budget_s / 3:
        n = min(n, cfg.T - done)
        tok = np.arange(done, done + n, dtype=np.int32)
        t0 = time.perf_counter()
        run(tok)
        t1 += time.perf_counter() - t0
        done += n
        n *= 2
    single = dict(value=done / t1, cores=1,
                  sample=f"tokens 0..{done - 1} of {cfg.T} ({t1:.1f} s)")
    nt = host_threads()
    rate1 = done / t1
    per = max(1, int(rate1 * budget_s * 2 / 3))   # tokens one thread does in the rest
    N = min(cfg.T, nt * per)
    nt = max(1, min(nt, N))
    blocks = [np.arange(N * i // nt, N * (i + 1) // nt, dtype=np.int32) for i in range(nt)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(run, blocks))
    tm = time.perf_counter() - t0
    return dict(value=N / tm, unit="tokens/s", cores=nt, kind="oracle",
                sample=f"tokens 0..{N - 1} of {cfg.T} of {cfg.name} in {nt} "
                       f"contiguous blocks, one host thread each ({tm:.1f} s wall; plain C, "
                       f"fp64 accumulation, forward only)",
                single_thread=single, cpu_model=cpu_model(), host_ram_gb=host_ram_gb())


# ------------------------------------------------------------------ PMC summary


def is_dominant(kernel_name: str, kind: str) -> bool:
    """The gate/up launch of the dominant kernel, demangled or mangled.
    Stream GEMM: template arguments <TW, XM, NSUB, EPI, KW, U, FR> with EPI =
    SwiGLU (1).  Tiled GEMM: <TBM, NM, EPI, GATHER, FR, CB> = <256, 2, 1, true,
    either weight layout, false>."""
    import re
    if DOMINANT[kind] not in kernel_name:
        return False
    if kind == "tiled":
        n = kernel_name.replace(" ", "")
        return bool(re.search(r"tiled_gemm_kernel<256,2,1,true(,(true|false))*>", n)
                    or "tiled_gemm_kernelILi256ELi2ELi1ELb1E" in n)
    n = kernel_name.replace(" ", "")
    m = re.search(r"stream_gemm_kernel<[^,]+,(\d+),(\d+),(\d+),", n)
    if m:
        return m.group(3) == "1"
    m = re.search(r"stream_gemm_kernelI(?:DF16_|f)Li(\d+)ELi(\d+)ELi(\d+)E", n)
    return bool(m) and m.group(3) == "1"


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str, copy_bytes: int, kind: str):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the dominant
    kernel, each scaled by what the counter reads for the calibration copy
    kernel of known size; writes profiles/traffic_...json."""
    import csv

    def read(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                rows += list(csv.DictReader(fh))
        dom, cp = [], []
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            v = float(r["Counter_Value"])
            if is_dominant(name, kind):
                dom.append(v)
            elif "AUnaryFunctor" in name and "MulFunctor" in name:  # the calibration copy
                cp.append(v)
        return dom, cp

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        dom, cp = read(d, counter)
        if not dom or not cp:
            raise SystemExit(f"no {counter} rows for the dominant or copy kernel in {d}")
        # the calibration copy reads and writes copy_bytes
        factor = copy_bytes / 1024.0 / statistics.median(cp)
        out[counter] = dict(kib_per_launch=statistics.median(dom), copy_kib=statistics.median(cp),
                            copy_factor=factor,
                            bytes_per_launch=statistics.median(dom) * 1024.0 * factor)
    what = "SwiGLU gate/up weight stream" if kind == "stream" else "SwiGLU gate/up, gathered rows"
    rec = dict(kernel=f"{DOMINANT[kind]} ({what})", workload=workload,
               kernel_source_hash=kernel_source_hash(kind), counters=out,
               traffic_bytes_per_launch=out["FETCH_SIZE"]["bytes_per_launch"]
               + out["WRITE_SIZE"]["bytes_per_launch"])
    rec["command"] = ("cd /tmp && rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv "
                      "-d DIR -o run -- python3 bench.py --workload N --steps 3 --warmup 1 "
                      "--no-cpu-baseline --no-prefill --copy-calibration; python3 bench.py "
                      "--summarize-pmc FETCH_DIR WRITE_DIR --workload N")
    p = traffic_path(kind, workload)
    with open(p, "w") as f:
        json.dump(rec, f, indent=2)
    print(json.dumps(rec, indent=2))


def kernel_label(name: str) -> str:
    """Short label of a libmoe kernel from its rocprofv3 name (demangled or
    mangled): the GEMM kind and epilogue, else the kernel's own name."""
    import re
    n = name.replace(" ", "")
    if "tiled_gemm_kernel" in n:
        m = re.search(r"tiled_gemm_kernel<(\d+),(\d+),(\d+),(true|false)", n) or re.search(
            r"tiled_gemm_kernelILi(\d+)ELi(\d+)ELi(\d+)ELb([01])E", n)
        if m:
            epi = {"0": "down", "1": "gate/up", "2": "router"}[m.group(3)]
            # the sixth argument: the combine in the launch's tail
            cb = re.search(r"tiled_gemm_kernel<[^>]*,(true|false),(true|false),true>", n) or \
                re.search(r"tiled_gemm_kernelI(?:[^E]*E){3}Lb[01]ELb[01]ELb1E", n)
            tail = " + combine in the tail" if cb else ""
            return f"tiled_gemm_kernel {epi} ({m.group(1)}-row tiles){tail}"
    if "stream_gemm_kernel" in n:
        m = re.search(r"stream_gemm_kernel<[^,]+,(\d+),(\d+),(\d+),", n) or re.search(
            r"stream_gemm_kernelI(?:DF16_|f)Li(\d+)ELi(\d+)ELi(\d+)E", n)
        if m:
            epi = {"0": "down", "1": "gate/up", "2": "router"}[m.group(3)]
            return f"stream_gemm_kernel {epi}"
    for k in ("topk_kernel", "dispatch_small_kernel", "dispatch_rank_kernel",
              "dispatch_place_kernel", "dispatch_scan_kernel", "dispatch_index_kernel",
              "dispatch_rows_kernel", "combine_kernel", "counts_kernel"):
        if k in n:
            return k
    return ""


def summarize_pmc_all(fetch_dir: str, write_dir: str, workload: str, copy_bytes: int):
    """FETCH_SIZE / WRITE_SIZE per launch of every libmoe kernel of the run
    (medians), scaled by the calibration copy; writes
    profiles/traffic_layer_kernels_<workload>.json."""
    import csv
    import collections

    out = collections.defaultdict(dict)
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals, cp = collections.defaultdict(list), []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r.get("Counter_Name") != counter:
                        continue
                    name = r.get("Kernel_Name", "")
                    v = float(r["Counter_Value"])
                    if "AUnaryFunctor" in name and "MulFunctor" in name:
                        cp.append(v)
                    elif kernel_label(name):
                        vals[kernel_label(name)].append(v)
        if not cp:
            raise SystemExit(f"no calibration copy rows for {counter} in {d}")
        factor = copy_bytes / 1024.0 / statistics.median(cp)
        for k, v in vals.items():
            out[k][counter + "_bytes"] = statistics.median(v) * 1024.0 * factor
            out[k][counter + "_launches"] = len(v)
        out["_copy_factor"][counter] = factor
    rec = dict(workload=workload, kernels=dict(out),
               command=("cd /tmp && rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format "
                        "csv -d DIR -o run -- python3 bench.py --workload N --steps 3 --warmup 1 "
                        "--no-cpu-baseline --no-prefill --copy-calibration; python3 bench.py "
                        "--summarize-pmc-all FETCH_DIR WRITE_DIR --workload N"))
    p = os.path.join(ROOT, "profiles", f"traffic_layer_kernels_{workload}.json")
    with open(p, "w") as f:
        json.dump(rec, f, indent=2)
    print(json.dumps(rec, indent=2))


def summarize_counters(pmc_dir: str):
    """Any rocprofv3 --pmc run: per libmoe kernel (kernel_label) and
    counter, the median value per launch and the launch count.  Used for
    the MFMA counters (MfmaFlopsF16 = SQ_INSTS_VALU_MFMA_MOPS_F16 x 512,
    MfmaUtil), which check the FLOPs the GEMMs execute against the
    algorithmic count."""
    import csv
    import collections
    vals = collections.defaultdict(list)
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                lab = kernel_label(r.get("Kernel_Name", ""))
                if lab:
                    vals[(lab, r.get("Counter_Name", ""))].append(float(r["Counter_Value"]))
    out = collections.defaultdict(dict)
    for (lab, counter), v in sorted(vals.items()):
        out[lab][counter] = {"median_per_launch": statistics.median(v), "launches": len(v)}
    print(json.dumps(out, indent=1))
    return dict(out)


def summarize_trace(trace_dir: str):
    """Per-kernel launch statistics of a rocprofv3 --kernel-trace run of
    this script: libmoe kernels grouped by name and grid (the same kernel
    serves launches of different shapes), split into the main workload and
    the prefill leg (which starts at the first LDS-tiled GEMM; the main
    workloads at decode sizes use none)."""
    import csv
    import collections
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    legs = collections.OrderedDict(main=[], prefill=[])
    leg = "main"
    for r in rows:
        lab = kernel_label(r["Kernel_Name"])
        if not lab:
            continue
        if "tiled_gemm_kernel" in lab:
            leg = "prefill"
        wg = int(r["Workgroup_Size_X"])
        grid = (int(r["Grid_Size_X"]) // max(wg, 1), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        legs[leg].append((lab, grid, r["Kernel_Name"], dur))
    out = {}
    for leg, ks in legs.items():
        g = collections.defaultdict(list)
        names = {}
        for lab, grid, name, dur in ks:
            g[(lab, grid)].append(dur)
            names[(lab, grid)] = name
        tot = sum(sum(v) for v in g.values())
        out[leg] = [dict(kernel=lab, grid=list(grid), name=names[(lab, grid)], calls=len(v),
                         avg_us=round(statistics.mean(v), 2),
                         median_us=round(statistics.median(v), 2),
                         share=round(sum(v) / tot, 4) if tot else 0.0)
                    for (lab, grid), v in sorted(g.items(), key=lambda kv: -sum(kv[1]))]
    print(json.dumps(out, indent=1))
    return out


# ------------------------------------------------------------------ context


def _timed(fn, flops, reps):
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"us": round(ms * 1e3, 1), "tflops": round(flops / (ms / 1e3) / 1e12, 1)}


def tiled_equal_groups(G, M, H, I, T, K, E, reps=10):
    """The library's own gate/up launch (moe_expert_ffn_up: the LDS-tiled
    kernel, rows gathered from h, SwiGLU epilogue, fragment-layout weights)
    on G equal groups of M rows -- the same flops and groups as the vendor
    comparison, without the ragged tails of routed groups.  Random operands
    (timing only)."""
    import numpy as np
    import torch

    import expert_router_gemm_amd as moe
    dev = "cuda:0"
    torch.manual_seed(0)
    rng = np.random.default_rng(0)
    wg = moe.pack_weights((torch.randn(G, I, H, device=dev) * 0.02).half())
    wu = moe.pack_weights((torch.randn(G, I, H, device=dev) * 0.02).half())
    h = torch.randn(T, H, device=dev).half()
    # each group gathers M distinct tokens in ascending order (as dispatch
    # orders a slot's rows); perm codes t * K + k
    gat = np.concatenate([np.sort(rng.choice(T, M, replace=False)) * K + (g % K)
                          for g in range(G)]).astype(np.int32)
    off = (np.arange(G + 1) * M).astype(np.int32)
    gather, offsets = torch.from_numpy(gat).to(dev), torch.from_numpy(off).to(dev)
    cap = T * K  # the layer's capacity (sizes the launch as in the layer)
    hm = torch.empty(cap, I, dtype=torch.float16, device=dev)
    shape = moe.make_shape(hidden=H, inter=I, n_experts=E, top_k=K, n_slots=G, act=moe.MOE_F16,
                           w_layout=moe.MOE_W_FRAG)
    r = _timed(lambda: moe.moe_expert_ffn_up(shape, G, cap, h, moe.MOE_F16, None,
                                             moe.MOE_X_GATHER, gather, offsets, wg, wu, hm),
               4 * G * M * H * I, reps)
    del wg, wu, h, hm
    torch.cuda.empty_cache()
    return r


def library_bmm(G, M, K, N, reps=10):
    """torch.bmm (hipBLASLt) fp16 on G groups of [M, K] x [K, N], contiguous."""
    import torch
    torch.manual_seed(0)
    a = torch.randn(G, M, K, device="cuda:0", dtype=torch.float16)
    b = torch.randn(G, K, N, device="cuda:0", dtype=torch.float16)
    r = _timed(lambda: torch.bmm(a, b), 2 * G * M * K * N, reps)
    del a, b
    torch.cuda.empty_cache()
    return r


def library_gemm(reps: int = 20):
    """For scale: torch's fp16 products (hipBLASLt) on the prefill expert
    GEMM shapes, contiguous operands: one [M, K] x [K, N] product and the
    same flops as 32 batched groups of 512 rows.  Not part of the layer."""
    import torch
    dev = "cuda:0"
    torch.manual_seed(0)

    def timed(fn, flops):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        return {"us": round(ms * 1e3, 1), "tflops": round(flops / (ms / 1e3) / 1e12, 1)}

    out = {}
    for (M, K, N) in [(16384, 7168, 4096), (16384, 2048, 7168), (8192, 8192, 8192)]:
        a = torch.randn(M, K, device=dev, dtype=torch.float16)
        b = torch.randn(K, N, device=dev, dtype=torch.float16)
        out[f"mm {M}x{K} @ {K}x{N}"] = timed(lambda: torch.mm(a, b), 2 * M * K * N)
    for (G, M, K, N) in [(32, 512, 7168, 4096), (32, 512, 2048, 7168)]:
        a = torch.randn(G, M, K, device=dev, dtype=torch.float16)
        b = torch.randn(G, K, N, device=dev, dtype=torch.float16)
        out[f"bmm {G}x[{M}x{K} @ {K}x{N}]"] = timed(lambda: torch.bmm(a, b), 2 * G * M * K * N)
    print(json.dumps({"library_gemm_fp16": out}))
    return out


# ------------------------------------------------------------------ main


def free_gpu(ctx):
    import torch
    ctx.clear()
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def prefill_record(K: int, warmup: int, w_layout: str = "frag", fused_combine: bool = False):
    """The prefill workload timed like the main one; tokens/s, the MFMA
    fraction of its gate/up launch and of the whole layer."""
    import torch

    import expert_router_gemm_amd as moe
    ctx = setup(PREFILL_WORKLOAD, keep_host=False, w_layout=w_layout,
                fused_combine=fused_combine)
    cfg = ctx["cfg"]
    t = time_workload(ctx, K, warmup, references=False)
    t["step_dist"] = step_distribution(ctx, K)
    prof_ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    profiled_step(ctx, moe.make_profile(prof_ev))
    torch.cuda.synchronize()
    names = ["route", "dispatch", "ffn_up", "ffn_down+shared", "combine"]
    t["stage_ms"] = {n: prof_ev[j].elapsed_time(prof_ev[j + 1]) for j, n in enumerate(names)}
    work = algorithmic_work(cfg, _counts_of(ctx))
    rec = {"workload": cfg.name, "tokens": cfg.T, "local_slots": ctx["S"],
           "weight_layout": LAYOUT_NAME[w_layout],
           "combine": COMBINE_NAME[fused_combine],
           "value": round(cfg.T / (t["ms_per_step"] / 1e3), 1), "unit": "tokens/s",
           "steps": K, "warmup": warmup, "ms_per_step": round(t["ms_per_step"], 4),
           "roofline": kernel_roofline(cfg, work, t["up_ms"], "tiled"),
           "layer": layer_record(work, t)}
    rec["layer"]["stage_ms_one_pass"] = {k: round(v, 4) for k, v in t["stage_ms"].items()}
    free_gpu(ctx)
    # context: the vendor library on the same gate/up flops, as uniform
    # contiguous groups (no gather, no ragged tail, no fused epilogue)
    # (equal groups holding this step's rows, and the same groups cut to a
    # multiple of 256 rows, the library's best case)
    G = cfg.E // cfg.ep_size  # local experts
    rows = -(-work["P"] // G)
    vendor, own = {}, {}
    for key, m in (("equal_groups", rows), ("aligned_groups", rows // 256 * 256)):
        if m <= 0:
            continue
        lib = library_bmm(G, m, cfg.H, 2 * cfg.I)
        vendor[key] = dict(lib, shape=f"{G} x [{m} x {cfg.H} @ {cfg.H} x {2 * cfg.I}]",
                           tiled_over_vendor=round(rec["roofline"]["achieved"] / lib["tflops"], 3))
        # and this library's gate/up launch on the same equal groups
        mine = tiled_equal_groups(G, m, cfg.H, cfg.I, cfg.T, cfg.K, cfg.E)
        own[key] = dict(mine, shape=vendor[key]["shape"],
                        frac_of_peak=round(mine["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                        over_vendor=round(mine["tflops"] / lib["tflops"], 3))
    rec["vendor_bmm_gate_up"] = vendor
    rec["tiled_gate_up_equal_groups"] = own
    return rec


def _counts_of(ctx):
    """Per-slot counts of the routing the timed steps produced (the staged
    route + dispatch on the same input)."""
    import torch

    import expert_router_gemm_amd as moe
    cfg, shape, d, b = ctx["cfg"], ctx["shape"], ctx["d"], ctx["b"]
    fp8 = cfg.dispatch == "fp8"
    moe.moe_route(shape, cfg.T, d["h"], d["wr"], d["bias"], b["idx"], b["tw"],
                  b["sg"] if cfg.n_shared else None, None, b["ws"])
    moe.moe_dispatch(shape, cfg.T, d["h"], b["idx"], ctx["smap"], b["xp"] if fp8 else None,
                     b["xs"] if fp8 else None, b["counts"], b["offsets"], b["perm"], b["inv"],
                     b["ws"])
    torch.cuda.synchronize()
    return b["counts"].cpu().numpy()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill workload's extra record")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (PMC scale)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="per-kernel launch statistics of a rocprofv3 --kernel-trace run")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="median per launch of every counter of a rocprofv3 --pmc run, per kernel")
    ap.add_argument("--summarize-pmc-all", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="per-kernel HBM traffic of every libmoe kernel of the two PMC runs")
    ap.add_argument("--eplb", action="store_true",
                    help="also report the EPLB-lite monitor cost and rank balance")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time torch's fp16 GEMMs on the prefill expert shapes")
    ap.add_argument("--w-layout", choices=["frag", "rowmajor"], default="frag",
                    help="expert weight layout: the fragment layout (default) or row-major")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the read probe and the vendor copy, sum and GEMM timed beside "
                         "the published peaks")
    ap.add_argument("--fused-combine", action="store_true",
                    help="set MOE_F_FUSED_COMBINE: the combine in the tiled down projection's "
                         "tail (prefill batches) instead of its own launch")
    ap.add_argument("--groups", metavar="G,M", default=None,
                    help="group-limited routing: keep M of G contiguous expert groups")
    args = ap.parse_args()
    groups = tuple(int(v) for v in args.groups.split(",")) if args.groups else None

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return 0
    if args.summarize_pmc_all:
        import moe_synth
        summarize_pmc_all(*args.summarize_pmc_all, moe_synth.config(args.workload).name, 1 << 30)
        return 0
    if args.summarize_pmc:
        import moe_synth
        summarize_pmc(*args.summarize_pmc, moe_synth.config(args.workload).name, 1 << 30,
                      dominant_kind(args.workload))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: expert parallelism across GPUs (the all-to-all "
              f"dispatch and combine) is not implemented (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.library_gemm:
        library_gemm()
        return 0
    import expert_router_gemm_amd as moe
    moe.lib()
    want_cpu = not args.no_cpu_baseline
    ctx = setup(args.workload, keep_host=want_cpu, groups=groups, w_layout=args.w_layout,
                fused_combine=args.fused_combine)
    cfg = ctx["cfg"]
    kind = dominant_kind(args.workload)

    t = time_workload(ctx, args.steps, args.warmup)
    log(f"[bench] timed {args.steps} steps of moe_layer_forward_profiled on {cfg.name}: "
        f"{t['ms_per_step']:.4f} ms/step, gate/up {t['up_ms'] * 1e3:.1f} us")
    work = algorithmic_work(cfg, ctx["b"]["counts"].cpu().numpy())
    value = cfg.T / (t["ms_per_step"] / 1e3)
    roof = kernel_roofline(cfg, work, t["up_ms"], kind)

    if args.copy_calibration:
        # a plain elementwise kernel that reads 1 GiB and writes 1 GiB
        a = torch.ones(1 << 29, dtype=torch.float16, device="cuda:0")
        bb = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=bb)
        torch.cuda.synchronize()
        del a, bb

    eplb = eplb_report(ctx) if args.eplb else None
    cpu = None
    if want_cpu:
        t0 = time.time()
        cpu = cpu_baseline(ctx, args.cpu_budget)
        log(f"[bench] cpu baseline: {cpu['value']:.2f} tokens/s on {cpu['cores']} threads, "
            f"{cpu['single_thread']['value']:.2f} on one ({time.time() - t0:.1f} s)")
    layer = layer_record(work, t)
    rec = {
        "metric": "MoE-layer tokens/s at 1 GPU + % HBM BW (decode) / % MFMA peak (prefill)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "f16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "inter": cfg.I,
                   "experts": cfg.E, "top_k": cfg.K, "local_slots": ctx["S"],
                   "shared_experts": cfg.n_shared, "dispatch": cfg.dispatch,
                   "ep_size": cfg.ep_size, "ep_rank": cfg.ep_rank,
                   "long_tail": cfg.long_tail,
                   "group_limit": list(groups) if groups else None,
                   "weight_layout": LAYOUT_NAME[args.w_layout],
                   "combine": COMBINE_NAME[args.fused_combine]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layer": layer,
    }
    if eplb:
        rec["eplb"] = eplb
    free_gpu(ctx)
    if not args.no_prefill and args.workload != PREFILL_WORKLOAD:
        rec["prefill"] = prefill_record(args.steps, args.warmup, args.w_layout,
                                        args.fused_combine)
        log(f"[bench] prefill {rec['prefill']['workload']}: {rec['prefill']['value']:.0f} "
            f"tokens/s, gate/up {rec['prefill']['roofline']['achieved']} TFLOP/s")
    if not args.no_reference:
        rec["reference"] = reference_rates()
        a = rec["reference"]
        probe = a["hbm_read_probe"]
        log(f"[bench] vendor kernels: copy {a['hbm']['copy_gbs']} GB/s, sum {a['hbm']['read_gbs']} "
            f"GB/s, fp16 GEMM {a['mfma']['tflops']} TFLOP/s; read probe "
            f"{probe['gbs'] if probe else 'not built'} GB/s")
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
