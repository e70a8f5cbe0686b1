"""ctypes front end of ``moe_oracle.c`` plus the oracle's own host logic.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pins (tests/test_oracle_pins.py) per function:
  router_logits   fp64 recomputation error bound; duplicate rows tie; bias
  softmax_topk    lexsort brute force; shift invariance; sum of all probs = 1;
                  group-limited: hand-worked cases, brute force over kept
                  groups + masked plain top-K, M = G reduces to plain
  shared_gate     w_sg = 0 gives exactly 0.5; closed form on tiny inputs
  slot_map        the blog page's worked example (section 2.2, Step 1);
                  replica choice against a Python SplitMix64 from the paper
  dispatch        stable argsort brute force; permutation invariants
  e4m3 codec      exhaustive round trip of all 256 codes; RNE midpoints;
                  torch.float8_e4m3fn on CPU after the clamp
  expert_rows     torch CPU SwiGLU reference in float64
  combine         closed forms (identical experts, dominant logit)
  layer_forward   numpy dense masked all-experts sum on tiny inputs;
                  top-k = E reduces to a dense softmax-weighted MoE
Parity unpinned (definitions, not results): the gate forms (softmax over all
logits without renormalisation, sigmoid shared gate), the replica hash and
the long-tail bias value.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Mutation tests point this at a deliberately broken build of the oracle to
# check that the pins catch it; normal use never sets it.
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB")

F32, F16 = 0, 1


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC",
                               "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            _lib = ctypes.CDLL(_LIB_OVERRIDE)
            _declare(_lib)
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "I", "E", "K", "S", "n_shared", "dtype", "fp8_dispatch",
                 "n_groups", "topk_groups")]


_p = ctypes.c_void_p
_i = ctypes.c_int
_u64 = ctypes.c_uint64


def _declare(L):
    L.oref_f16_to_double.argtypes = [ctypes.c_uint16]
    L.oref_f16_to_double.restype = ctypes.c_double
    L.oref_router_logits.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p]
    L.oref_softmax_topk.argtypes = [_i, _i, _i, _p, _p, _p]
    L.oref_softmax_topk_grouped.argtypes = [_i, _i, _i, _i, _i, _p, _p, _p]
    L.oref_shared_gate.argtypes = [_i, _i, _i, _p, _p, _p]
    L.oref_splitmix64.argtypes = [_u64]
    L.oref_splitmix64.restype = _u64
    L.oref_slot_map.argtypes = [_i, _i, _p, _p, _p, _p, _u64, _p]
    L.oref_dispatch.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p]
    L.oref_e4m3_encode.argtypes = [ctypes.c_float]
    L.oref_e4m3_encode.restype = ctypes.c_uint8
    L.oref_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.oref_e4m3_decode.restype = ctypes.c_float
    L.oref_quant_e4m3_rows.argtypes = [_i, _i, _i, _p, _p, _p]
    L.oref_expert_rows.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p]
    L.oref_combine.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p]
    L.oref_layer_forward.argtypes = [ctypes.POINTER(Dims), _p, _p, _p, _p, _p,
                                     _p, _p, _p, _p, _p, _p, _p, _p, _u64,
                                     _p, _p, _p, _p, _p, _p]
    L.oref_layer_forward.restype = _i


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"unsupported dtype {a.dtype}")


def _c(a, dtype=None):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- stages


def router_logits(h: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """Step 1 router linear: fp32 logits [T, E] (fp64 dot products)."""
    h = _c(h)
    w_router = _c(w_router, h.dtype)
    T, H = h.shape
    E = w_router.shape[0]
    out = np.empty((T, E), np.float32)
    lib().oref_router_logits(T, H, E, _dt(h), _ptr(h), _ptr(w_router),
                             _ptr(_c(bias, np.float32)), _ptr(out))
    return out


def softmax_topk(logits: np.ndarray, K: int, groups=None):
    """Softmax over all experts, top-K by (logit desc, id asc).  groups =
    (G, M): group-limited routing (M of G contiguous groups, by their best
    logit), see oref_softmax_topk_grouped."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    if groups:
        G, M = groups
        lib().oref_softmax_topk_grouped(T, E, K, G, M, _ptr(logits), _ptr(idx), _ptr(w))
    else:
        lib().oref_softmax_topk(T, E, K, _ptr(logits), _ptr(idx), _ptr(w))
    return idx, w


def shared_gate(h: np.ndarray, w_sg: np.ndarray) -> np.ndarray:
    h = _c(h)
    w_sg = _c(w_sg, h.dtype)
    T, H = h.shape
    out = np.empty(T, np.float32)
    lib().oref_shared_gate(T, H, _dt(h), _ptr(h), _ptr(w_sg), _ptr(out))
    return out


def splitmix64(x: int) -> int:
    return int(lib().oref_splitmix64(x))


def slot_map(topk_idx, rep_off, rep_slot, seed: int, tok_ids=None) -> np.ndarray:
    topk_idx = _c(topk_idx, np.int32)
    T, K = topk_idx.shape
    out = np.empty((T, K), np.int32)
    lib().oref_slot_map(T, K, _ptr(topk_idx), _ptr(_c(tok_ids, np.int32)),
                        _ptr(_c(rep_off, np.int32)), _ptr(_c(rep_slot, np.int32)),
                        seed, _ptr(out))
    return out


def dispatch(slot: np.ndarray, S: int):
    """Step 2 as a stable counting sort: (counts, offsets, perm_src, inv_pos)."""
    slot = _c(slot, np.int32)
    T, K = slot.shape
    counts = np.empty(S, np.int32)
    offsets = np.empty(S + 1, np.int32)
    perm = np.full(max(T * K, 1), -1, np.int32)
    inv = np.empty((T, K), np.int32)
    lib().oref_dispatch(T, K, S, _ptr(slot), _ptr(counts), _ptr(offsets),
                        _ptr(perm), _ptr(inv))
    return counts, offsets, perm[: int(offsets[S])].copy(), inv


def e4m3_encode(v: float) -> int:
    return int(lib().oref_e4m3_encode(float(v)))


def e4m3_decode(c: int) -> float:
    return float(lib().oref_e4m3_decode(int(c)))


def e4m3_decode_table() -> np.ndarray:
    return np.array([e4m3_decode(c) for c in range(256)], np.float32)


def quant_e4m3_rows(x: np.ndarray):
    """Per-row fp8 e4m3 codes [R, H] (uint8) and fp32 scales [R]."""
    x = _c(x)
    R, H = x.shape
    q = np.empty((R, H), np.uint8)
    s = np.empty(R, np.float32)
    lib().oref_quant_e4m3_rows(R, H, _dt(x), _ptr(x), _ptr(q), _ptr(s))
    return q, s


def expert_rows(x: np.ndarray, wg, wu, wd, want_hm: bool = False):
    """Step 3 SwiGLU on rows x [R, H] (any float dtype; used as float64)."""
    x = _c(x, np.float64)
    wg = _c(wg)
    dt = _dt(wg)
    wu = _c(wu, wg.dtype)
    wd = _c(wd, wg.dtype)
    R, H = x.shape
    I = wg.shape[0]
    y = np.empty((R, H), np.float32)
    hm = np.empty((R, I), np.float32) if want_hm else None
    lib().oref_expert_rows(R, H, I, dt, _ptr(x), _ptr(wg), _ptr(wu), _ptr(wd),
                           _ptr(hm), _ptr(y))
    return (y, hm) if want_hm else y


def combine(y, inv_pos, topk_w, shared_y=None, shared_gate_v=None, H=None):
    """Steps 4-5: gate-weighted sum (+ gated sum of shared experts).

    y [P, H] (P may be 0: no local pair); H is y's row length, or that of
    shared_y, unless given."""
    y = _c(y, np.float32)
    inv_pos = _c(inv_pos, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, K = inv_pos.shape
    if H is None:
        H = y.shape[1] if y.ndim == 2 else (shared_y.shape[-1] if shared_y is not None else 0)
    n_sh = 0 if shared_y is None else shared_y.shape[0]
    out = np.empty((T, H), np.float32)
    if y.size == 0:
        y = np.zeros((1, max(H, 1)), np.float32)
    lib().oref_combine(T, K, H, n_sh, _ptr(y), _ptr(inv_pos), _ptr(topk_w),
                       _ptr(_c(shared_y, np.float32)),
                       _ptr(_c(shared_gate_v, np.float32)), _ptr(out))
    return out


# ---------------------------------------------------------------- placement


def placement(E: int, ep_size: int, ep_rank: int, replica_of: Optional[int] = None):
    """Expert -> local-slot table for one GPU of an EP group.

    Blog page section 2.1: with EP = N each GPU holds a contiguous 1/N of the
    routed experts (GPU g holds E/N*g .. E/N*(g+1)-1), so expert e lives on GPU
    e // (E/N).  Section 6.3: a redundant copy of a hot expert can sit on a
    second GPU; reading taken here: the copy becomes one extra local slot after
    the resident ones, and the expert's replica list is [home copy, extra slot]
    (the home copy is -1 when it lives on another GPU).

    Returns (rep_off [E+1], rep_slot [nnz], slot_experts [S]).
    """
    per = E // ep_size
    rep_off = [0]
    rep_slot = []
    slot_experts = list(range(ep_rank * per, (ep_rank + 1) * per))
    extra = None
    if replica_of is not None:
        extra = len(slot_experts)
        slot_experts.append(replica_of)
    for e in range(E):
        home = e // per
        rep_slot.append(e - ep_rank * per if home == ep_rank else -1)
        if replica_of is not None and e == replica_of:
            rep_slot.append(extra)
        rep_off.append(len(rep_slot))
    return (np.array(rep_off, np.int32), np.array(rep_slot, np.int32),
            np.array(slot_experts, np.int32))


def gpu_of_expert(e: int, E: int = 256, ep_size: int = 8) -> int:
    """Which GPU of the EP group holds expert e (contiguous placement)."""
    return e // (E // ep_size)


# ---------------------------------------------------------------- layer


def layer_forward(*, h: np.ndarray, w_router: np.ndarray, bias, w_sg,
                  slot_weights: Sequence, shared: Optional[Sequence],
                  rep_off, rep_slot, seed: int, K: int, fp8_dispatch: bool,
                  tok_ids=None, I: Optional[int] = None, groups=None):
    """Whole-layer oracle (Steps 1-5) for the tokens in ``h``.

    slot_weights: list over local slots of (gate [I,H], up [I,H], down [H,I])
    tuples or None (weights not supplied; an error if a pair lands there).
    shared: (gate [n,I,H], up [n,I,H], down [n,H,I]) or None.
    groups: (G, M) for group-limited routing, or None.
    Returns dict(out, topk_idx, topk_w, slot, logits, shared_gate).
    """
    h = _c(h)
    T, H = h.shape
    dt = _dt(h)
    E = w_router.shape[0]
    S = len(slot_weights)
    if I is None:
        for sw in slot_weights:
            if sw is not None:
                I = sw[0].shape[0]
                break
        if I is None and shared is not None:
            I = shared[0].shape[1]
    I = int(I or 0)
    n_sh = 0 if shared is None else int(shared[0].shape[0])
    G, M = groups if groups else (0, 0)
    d = Dims(T, H, I, E, K, S, n_sh, dt, 1 if fp8_dispatch else 0, G, M)
    keep = []

    def arr(ptrs):
        a = (ctypes.c_void_p * max(S, 1))()
        for i, p in enumerate(ptrs):
            a[i] = p
        return a

    gp, up, dp = [], [], []
    for sw in slot_weights:
        if sw is None:
            gp.append(None), up.append(None), dp.append(None)
            continue
        g, u, dd = (_c(m, h.dtype) for m in sw)
        keep += [g, u, dd]
        gp.append(g.ctypes.data), up.append(u.ctypes.data), dp.append(dd.ctypes.data)
    sh = [None, None, None]
    if shared is not None:
        sh = [_c(m, h.dtype) for m in shared]
    w_router = _c(w_router, h.dtype)
    w_sg = _c(w_sg, h.dtype)
    out = np.empty((T, H), np.float32)
    idx = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    slot = np.empty((T, K), np.int32)
    logits = np.empty((T, E), np.float32)
    gs = np.empty(T, np.float32)
    rc = lib().oref_layer_forward(
        ctypes.byref(d), _ptr(h), _ptr(_c(tok_ids, np.int32)), _ptr(w_router),
        _ptr(_c(bias, np.float32)), _ptr(w_sg), arr(gp), arr(up), arr(dp),
        _ptr(sh[0]), _ptr(sh[1]), _ptr(sh[2]), _ptr(_c(rep_off, np.int32)),
        _ptr(_c(rep_slot, np.int32)), seed, _ptr(out), _ptr(idx), _ptr(w),
        _ptr(slot), _ptr(logits), _ptr(gs))
    if rc == -2:
        raise ValueError("oracle: two pairs of one token land in one slot (a token's experts "
                         "are distinct and a slot holds one expert)")
    if rc != 0:
        raise RuntimeError("oracle: a pair was routed to a slot without weights")
    return dict(out=out, topk_idx=idx, topk_w=w, slot=slot, logits=logits,
                shared_gate=gs if n_sh else None)


def near_tie_tokens(logits: np.ndarray, K: int, gap: float = 1e-5) -> np.ndarray:
    """Tokens whose top-(K+1) sorted logits have an adjacent gap < ``gap``.

    On such tokens two correct implementations that round their sums in a
    different order may legitimately select different experts."""
    s = -np.sort(-logits.astype(np.float64), axis=1)[:, : K + 1]
    return np.any(np.abs(np.diff(s, axis=1)) < gap, axis=1)
