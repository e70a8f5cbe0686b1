"""GPU-side helpers for the parity tests: upload seeded inputs, run libmoe
through its C ABI (the Python binding), and run the oracle on the same data.

The HIP path and the oracle share only moe_synth (the seeded inputs).  Each
side builds its own expert -> slot table (expert_router_gemm_amd.placement
vs oracle.placement; a CPU test checks they agree).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import expert_router_gemm_amd as moe
import moe_synth
import oracle

DEV = "cuda:0"

# Stated tolerance on layer outputs (fp16 outputs, fp32 accumulation).
ATOL, RTOL = 2e-3, 2e-2

# Expert weights are uploaded in the layout the benchmark runs (the
# fragment layout); tests of the row-major layout ask for it explicitly.
DEFAULT_W_LAYOUT = moe.MOE_W_FRAG


def within_tol(gpu, ref, atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(gpu - ref) <= atol + rtol * np.abs(ref)


def assert_close(gpu, ref, what, atol=ATOL, rtol=RTOL, rows=None):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    if rows is not None:
        gpu, ref = gpu[rows], ref[rows]
    ok = within_tol(gpu, ref, atol, rtol)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        err = np.abs(gpu - ref)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside |d| <= {atol} + "
                             f"{rtol}|ref|; max |d| = {err.max():.3e}; first bad {bad.tolist()} "
                             f"gpu={gpu[tuple(bad[0])]:.6g} ref={ref[tuple(bad[0])]:.6g}")
    return float(np.abs(gpu - ref).max()) if gpu.size else 0.0


def to_dev(a: Optional[np.ndarray]):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def act_code(cfg) -> int:
    return moe.MOE_F32 if cfg.dtype == "f32" else moe.MOE_F16


@dataclasses.dataclass
class Layer:
    cfg: object
    shape: object
    h: np.ndarray
    wr: np.ndarray
    bias: Optional[np.ndarray]
    slot_experts: np.ndarray
    rep_off: np.ndarray
    rep_slot: np.ndarray
    seed: int
    d: dict            # device tensors
    wmap: object       # moe.Weights
    smap: object       # moe.SlotMap
    experts: dict      # logical expert -> (g, u, d) host arrays (lazily filled)
    shared: Optional[tuple]
    rank: int

    @property
    def T(self):
        return self.h.shape[0]

    def expert(self, e):
        if e not in self.experts:
            self.experts[e] = moe_synth.gen_expert(self.cfg, int(e))
        return self.experts[e]


def build_layer(cfg, *, rank: Optional[int] = None, T: Optional[int] = None,
                bias_override: Optional[np.ndarray] = None, keep_host_weights=True,
                slot_seed: Optional[int] = None, w_layout: Optional[int] = None) -> Layer:
    """Generate the workload's inputs and upload them.

    rank: which EP rank this GPU plays (default: the workload's own).
    w_layout: MOE_W_FRAG (default; packed on the device by moe_pack_weights)
    or MOE_W_ROWMAJOR for the expert weights; host copies stay row-major."""
    w_layout = DEFAULT_W_LAYOUT if w_layout is None else w_layout
    rank = cfg.ep_rank if rank is None else rank
    rep = moe_synth.replica_expert(cfg)
    rep_off, rep_slot, slot_experts = moe.build_slot_map(cfg.E, cfg.ep_size, rank,
                                                         [rep] if rep is not None else None)
    h = moe_synth.gen_hidden(cfg, T)
    wr = moe_synth.gen_router(cfg)
    bias = moe_synth.gen_router_bias(cfg) if bias_override is None else bias_override
    S = len(slot_experts)
    dt = np.float32 if cfg.dtype == "f32" else np.float16
    tdt = torch.float32 if cfg.dtype == "f32" else torch.float16
    G = torch.empty((S, cfg.I, cfg.H), dtype=tdt, device=DEV)
    U = torch.empty((S, cfg.I, cfg.H), dtype=tdt, device=DEV)
    D = torch.empty((S, cfg.H, cfg.I), dtype=tdt, device=DEV)
    experts = {}
    for s, (e, (g, u, dd)) in enumerate(moe_synth.iter_experts(cfg, slot_experts)):
        G[s].copy_(torch.from_numpy(g))
        U[s].copy_(torch.from_numpy(u))
        D[s].copy_(torch.from_numpy(dd))
        if keep_host_weights:
            experts[e] = (g, u, dd)
    shared = None
    d = dict(h=to_dev(h), wr=to_dev(wr), bias=to_dev(bias), G=G, U=U, D=D)
    if cfg.n_shared:
        shared = moe_synth.gen_shared_weights(cfg)
        d.update(SG=to_dev(shared[0]), SU=to_dev(shared[1]), SD=to_dev(shared[2]))
    d.update(rep_off=to_dev(rep_off), rep_slot=to_dev(rep_slot))
    if w_layout == moe.MOE_W_FRAG:
        for k in ("G", "U", "D", "SG", "SU", "SD"):
            if k in d:
                d[k] = moe.pack_weights(d[k])  # the row-major copy is freed
        G, U, D = d["G"], d["U"], d["D"]
        torch.cuda.synchronize()
    shape = moe.make_shape(hidden=cfg.H, inter=cfg.I, n_experts=cfg.E, top_k=cfg.K, n_slots=S,
                           n_shared=cfg.n_shared, act=act_code(cfg),
                           dispatch=moe.MOE_FP8_E4M3 if cfg.dispatch == "fp8" else None,
                           shared=cfg.n_shared > 0, n_groups=cfg.n_groups,
                           topk_groups=cfg.topk_groups, w_layout=w_layout)
    wmap = moe.make_weights(w_router=d["wr"], bias=d["bias"], w_gate=G, w_up=U, w_down=D,
                            sh_gate=d.get("SG"), sh_up=d.get("SU"), sh_down=d.get("SD"))
    seed = cfg.seed if slot_seed is None else slot_seed
    smap = moe.make_slot_map(d["rep_off"], d["rep_slot"], seed)
    _ = dt
    return Layer(cfg, shape, h, wr, bias, slot_experts, rep_off, rep_slot, seed, d, wmap, smap,
                 experts, shared, rank)


def ws_for(L: Layer, T=None):
    T = L.T if T is None else T
    n = moe.moe_workspace_bytes(L.shape, T)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def gpu_forward(L: Layer, fused_combine: bool = False):
    """moe_layer_forward; fused_combine sets MOE_F_FUSED_COMBINE."""
    T, H = L.T, L.cfg.H
    out = torch.empty((T, H), dtype=L.d["h"].dtype, device=DEV)
    ws = ws_for(L)
    shape = L.shape
    if fused_combine:
        shape = type(L.shape).from_buffer_copy(L.shape)
        shape.flags |= moe.MOE_F_FUSED_COMBINE
    moe.moe_layer_forward(shape, L.wmap, L.smap, T, L.d["h"], out, ws)
    torch.cuda.synchronize()
    return out


def gpu_stages(L: Layer):
    """Run the staged entry points; return every intermediate (host copies)."""
    cfg = L.cfg
    T, K, H, I, E, S = L.T, cfg.K, cfg.H, cfg.I, cfg.E, len(L.slot_experts)
    dev = DEV
    act = L.d["h"].dtype
    ws = ws_for(L)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    tw = torch.empty((T, K), dtype=torch.float32, device=dev)
    sg = torch.empty((max(T, 1),), dtype=torch.float32, device=dev) if cfg.n_shared else None
    lg = torch.empty((T, E), dtype=torch.float32, device=dev)
    moe.moe_route(L.shape, T, L.d["h"], L.d["wr"], L.d["bias"], idx, tw, sg, lg, ws)
    fp8 = cfg.dispatch == "fp8"
    xp = torch.empty((max(T * K, 1), H), dtype=torch.uint8 if fp8 else act, device=dev)
    xs = torch.empty((max(T * K, 1),), dtype=torch.float32, device=dev)
    counts = torch.empty((S,), dtype=torch.int32, device=dev)
    offsets = torch.empty((S + 1,), dtype=torch.int32, device=dev)
    perm = torch.full((max(T * K, 1),), -7, dtype=torch.int32, device=dev)
    inv = torch.empty((T, K), dtype=torch.int32, device=dev)
    moe.moe_dispatch(L.shape, T, L.d["h"], idx, L.smap, xp, xs if fp8 else None, counts,
                     offsets, perm, inv, ws)
    cap = T * K
    hm = torch.empty((max(cap, 1), I), dtype=act, device=dev)
    y = torch.empty((max(cap, 1), H), dtype=act, device=dev)
    xdt = moe.MOE_FP8_E4M3 if fp8 else act_code(cfg)
    moe.moe_expert_ffn_up(L.shape, S, cap, xp, xdt, xs if fp8 else None, moe.MOE_X_PERMUTED,
                          None, offsets, L.d["G"], L.d["U"], hm)
    hm_gather = None
    if not fp8:  # the same rows gathered straight from h must give the same hm
        hm_gather = torch.empty_like(hm)
        moe.moe_expert_ffn_up(L.shape, S, cap, L.d["h"], act_code(cfg), None, moe.MOE_X_GATHER,
                              perm, offsets, L.d["G"], L.d["U"], hm_gather)
    moe.moe_expert_ffn_down(L.shape, S, cap, hm, offsets, L.d["D"], y)
    shy = None
    if cfg.n_shared:
        shoff = to_dev(np.arange(cfg.n_shared + 1, dtype=np.int32) * T)
        shy = torch.empty((cfg.n_shared * T, H), dtype=act, device=dev)
        moe.moe_expert_ffn(L.shape, cfg.n_shared, cfg.n_shared * T, L.d["h"], act_code(cfg),
                           None, moe.MOE_X_SHARED, None, shoff, L.d["SG"], L.d["SU"], L.d["SD"],
                           shy, ws)
    out = torch.empty((T, H), dtype=act, device=dev)
    moe.moe_combine(L.shape, T, y, inv, tw, shy, sg, out)
    torch.cuda.synchronize()
    P = int(offsets[S].item())
    host = lambda t: None if t is None else t.cpu().numpy()  # noqa: E731
    return dict(topk_idx=host(idx), topk_w=host(tw), shared_gate=host(sg), logits=host(lg),
                x_perm=host(xp[:P]), x_scale=host(xs[:P]) if fp8 else None, counts=host(counts),
                offsets=host(offsets), perm_src=host(perm[:P]), inv_pos=host(inv),
                hm=host(hm[:P]), y=host(y[:P]), shared_y=host(shy), out=host(out), P=P,
                hm_gather=None if hm_gather is None else host(hm_gather[:P]),
                perm_tail=host(perm[P:]))


def oracle_forward(L: Layer, tokens: Optional[np.ndarray] = None):
    """Oracle layer output for all tokens or a sample (global ids kept for
    the replica hash).  Regenerates only the experts it needs."""
    cfg = L.cfg
    h = L.h if tokens is None else np.ascontiguousarray(L.h[tokens])
    tok_ids = None if tokens is None else np.asarray(tokens, np.int32)
    rep = moe_synth.replica_expert(cfg)
    ro, rs, se = oracle.placement(cfg.E, cfg.ep_size, L.rank, replica_of=rep)
    # which slots will be touched: route this sample first
    lg = oracle.router_logits(h, L.wr[: cfg.E], L.bias)
    idx, _ = oracle.softmax_topk(lg, cfg.K, groups=cfg.groups)
    slot = oracle.slot_map(idx, ro, rs, L.seed, tok_ids=tok_ids)
    need = set(int(s) for s in np.unique(slot) if s >= 0)
    missing = [int(se[s]) for s in sorted(need) if int(se[s]) not in L.experts]
    for e, w in moe_synth.iter_experts(cfg, missing):
        L.experts[e] = w
    sw = [L.expert(se[s]) if s in need else None for s in range(len(se))]
    res = oracle.layer_forward(h=h, w_router=L.wr[: cfg.E], bias=L.bias,
                               w_sg=L.wr[cfg.E] if cfg.n_shared else None, slot_weights=sw,
                               shared=L.shared, rep_off=ro, rep_slot=rs, seed=L.seed, K=cfg.K,
                               fp8_dispatch=cfg.dispatch == "fp8", tok_ids=tok_ids,
                               groups=cfg.groups)
    return res


def logit_error_bound(L: Layer, tokens=None):
    """Deterministic bound on |gpu - exact| for fp32-accumulated logits:
    n * u * sum_i |h_i w_i| (u = 2^-24; the fp64 oracle is exact to far
    better), plus one rounding of the result."""
    cfg = L.cfg
    h = L.h if tokens is None else L.h[tokens]
    a = np.abs(h.astype(np.float64)) @ np.abs(L.wr[: cfg.E].astype(np.float64)).T
    return cfg.H * 2.0 ** -24 * a + 2.0 ** -22 * (a + 8.0)
