"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every function has the C name and argument order of the ABI; torch tensors
are passed as device pointers, ``stream=None`` means torch's current stream.
A non-OK status raises ``MoEError``.  The library must have been built
(``python -m expert_router_gemm_amd.build``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_F16, MOE_FP8_E4M3 = 0, 1, 2
MOE_F_SHARED = 1
MOE_F_FUSED_COMBINE = 2
MOE_X_PERMUTED, MOE_X_SHARED, MOE_X_GATHER = 0, 1, 2
MOE_W_ROWMAJOR, MOE_W_FRAG = 0, 1

EXPORTED = (
    "moe_route", "moe_dispatch", "moe_expert_ffn_up", "moe_expert_ffn_down",
    "moe_expert_ffn", "moe_combine", "moe_layer_forward", "moe_layer_forward_profiled",
    "moe_layer_forward_noalloc", "moe_pack_weights",
    "moe_workspace_bytes", "moe_status_str", "moe_version", "moe_expert_counts",
    "moe_eplb_state_bytes", "moe_eplb_init", "moe_eplb_observe", "moe_eplb_loads",
    "moe_eplb_rebalance", "moe_eplb_slot_map", "moe_eplb_cleanup",
)
_HOST_ONLY = ("moe_workspace_bytes", "moe_status_str", "moe_version", "moe_eplb_state_bytes")


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("act", ctypes.c_int32), ("dispatch", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("w_layout", ctypes.c_int32)]

    def __repr__(self):
        return "Shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class SlotMap(ctypes.Structure):
    _fields_ = [("rep_off", ctypes.c_void_p), ("rep_slot", ctypes.c_void_p),
                ("seed", ctypes.c_uint64)]


class Profile(ctypes.Structure):
    _fields_ = [("events", ctypes.c_void_p * 6)]


class EplbConfig(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("n_ranks", ctypes.c_int32),
                ("window", ctypes.c_int32), ("max_moves", ctypes.c_int32),
                ("spare_slots", ctypes.c_int32), ("threshold", ctypes.c_double)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "bias", "w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libmoe.so not found at {LIB_PATH}; build it with "
                "`python -m expert_router_gemm_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_uint64
        SP = ctypes.POINTER(Shape)
        L.moe_route.argtypes = [SP, I32, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_dispatch.argtypes = [SP, I32, P, P, ctypes.POINTER(SlotMap), P, P, P, P, P, P, P, SZ, P]
        L.moe_expert_ffn_up.argtypes = [SP, I32, I32, P, I32, P, I32, P, P, P, P, P, P]
        L.moe_expert_ffn_down.argtypes = [SP, I32, I32, P, P, P, P, P]
        L.moe_expert_ffn.argtypes = [SP, I32, I32, P, I32, P, I32, P, P, P, P, P, P, P, SZ, P]
        L.moe_combine.argtypes = [SP, I32, P, P, P, P, P, P, P]
        L.moe_layer_forward.argtypes = [SP, ctypes.POINTER(Weights), ctypes.POINTER(SlotMap),
                                        I32, P, P, P, SZ, P]
        L.moe_layer_forward_profiled.argtypes = [SP, ctypes.POINTER(Weights),
                                                 ctypes.POINTER(SlotMap), I32, P, P, P, SZ,
                                                 ctypes.POINTER(Profile), P]
        L.moe_layer_forward_noalloc.argtypes = [SP, ctypes.POINTER(Weights),
                                                ctypes.POINTER(SlotMap), I32, P, P, P]
        L.moe_workspace_bytes.argtypes = [SP, I32]
        L.moe_pack_weights.argtypes = [I32, ctypes.c_int64, I32, I32, P, P, P]
        L.moe_workspace_bytes.restype = SZ
        L.moe_expert_counts.argtypes = [SP, I32, P, P, P]
        EP = ctypes.POINTER(EplbConfig)
        L.moe_eplb_state_bytes.argtypes = [EP]
        L.moe_eplb_state_bytes.restype = SZ
        L.moe_eplb_init.argtypes = [EP, P, SZ]
        L.moe_eplb_observe.argtypes = [P, P]
        L.moe_eplb_loads.argtypes = [P, P, P]
        L.moe_eplb_rebalance.argtypes = [P, P, P]
        L.moe_eplb_slot_map.argtypes = [P, I32, P, P, P, P]
        L.moe_eplb_cleanup.argtypes = [P, I32, P, P]
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_version.restype = ctypes.c_char_p
        for fn in EXPORTED:
            if fn not in _HOST_ONLY:
                getattr(L, fn).restype = ctypes.c_int
        _ = U64
        _lib = L
    return _lib


def status_str(st: int) -> str:
    return lib().moe_status_str(int(st)).decode()


def version() -> str:
    return lib().moe_version().decode()


def _p(t) -> Optional[int]:
    """Device pointer of a tensor (or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(fn: str, st: int):
    if st != 0:
        raise MoEError(fn, st)


def make_shape(*, hidden, inter, n_experts, top_k, n_slots, n_shared=0, act=MOE_F16,
               dispatch=None, shared=False, n_groups=0, topk_groups=0,
               w_layout=MOE_W_ROWMAJOR, fused_combine=False) -> Shape:
    flags = (MOE_F_SHARED if shared else 0) | (MOE_F_FUSED_COMBINE if fused_combine else 0)
    return Shape(hidden, inter, n_experts, top_k, n_slots, n_shared, act,
                 act if dispatch is None else dispatch, flags, n_groups, topk_groups, w_layout)


def moe_workspace_bytes(shape: Shape, T: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape), T))


def moe_route(shape, T, h, w_router, bias, topk_idx, topk_w, shared_gate, logits, ws, stream=None):
    _check("moe_route", lib().moe_route(
        ctypes.byref(shape), T, _p(h), _p(w_router), _p(bias), _p(topk_idx), _p(topk_w),
        _p(shared_gate), _p(logits), _p(ws), _nbytes(ws), _stream(stream)))


def moe_dispatch(shape, T, h, topk_idx, slot_map: SlotMap, x_perm, x_scale, counts, offsets,
                 perm_src, inv_pos, ws, stream=None):
    _check("moe_dispatch", lib().moe_dispatch(
        ctypes.byref(shape), T, _p(h), _p(topk_idx), ctypes.byref(slot_map), _p(x_perm),
        _p(x_scale), _p(counts), _p(offsets), _p(perm_src), _p(inv_pos), _p(ws), _nbytes(ws),
        _stream(stream)))


def moe_expert_ffn_up(shape, n_groups, cap_rows, x, x_dtype, x_scale, x_rows, gather, offsets,
                      w_gate, w_up, hm, stream=None):
    _check("moe_expert_ffn_up", lib().moe_expert_ffn_up(
        ctypes.byref(shape), n_groups, cap_rows, _p(x), x_dtype, _p(x_scale), int(x_rows),
        _p(gather), _p(offsets), _p(w_gate), _p(w_up), _p(hm), _stream(stream)))


def moe_expert_ffn_down(shape, n_groups, cap_rows, hm, offsets, w_down, y, stream=None):
    _check("moe_expert_ffn_down", lib().moe_expert_ffn_down(
        ctypes.byref(shape), n_groups, cap_rows, _p(hm), _p(offsets), _p(w_down), _p(y),
        _stream(stream)))


def moe_expert_ffn(shape, n_groups, cap_rows, x, x_dtype, x_scale, x_rows, gather, offsets,
                   w_gate, w_up, w_down, y, ws, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        ctypes.byref(shape), n_groups, cap_rows, _p(x), x_dtype, _p(x_scale), int(x_rows),
        _p(gather), _p(offsets), _p(w_gate), _p(w_up), _p(w_down), _p(y), _p(ws), _nbytes(ws),
        _stream(stream)))


def moe_combine(shape, T, y, inv_pos, topk_w, shared_y, shared_gate, out, stream=None):
    _check("moe_combine", lib().moe_combine(
        ctypes.byref(shape), T, _p(y), _p(inv_pos), _p(topk_w), _p(shared_y), _p(shared_gate),
        _p(out), _stream(stream)))


def moe_layer_forward(shape, weights: Weights, slot_map: SlotMap, T, h, out, ws, stream=None):
    _check("moe_layer_forward", lib().moe_layer_forward(
        ctypes.byref(shape), ctypes.byref(weights), ctypes.byref(slot_map), T, _p(h), _p(out),
        _p(ws), _nbytes(ws), _stream(stream)))


def moe_layer_forward_noalloc(shape, weights: Weights, slot_map: SlotMap, T, h, out,
                              stream=None):
    """moe_layer_forward with the library's own static device workspace
    (for callers that cannot allocate; see include/moe.h)."""
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        ctypes.byref(shape), ctypes.byref(weights), ctypes.byref(slot_map), T, _p(h), _p(out),
        _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_pack_weights(dtype, n_mats, rows, cols, src, dst, stream=None):
    _check("moe_pack_weights", lib().moe_pack_weights(
        int(dtype), int(n_mats), int(rows), int(cols), _p(src), _p(dst), _stream(stream)))


def pack_weights(w, stream=None):
    """MOE_W_FRAG copy of the row-major expert weights ``w`` (fp16 or fp32,
    [..., rows, cols]); the result has w's shape and dtype."""
    import torch
    dtype = {torch.float16: MOE_F16, torch.float32: MOE_F32}.get(w.dtype)
    if dtype is None:
        raise ValueError("pack_weights takes fp16 or fp32 weights")
    if w.dim() < 2:
        raise ValueError("pack_weights takes [..., rows, cols]")
    rows, cols = w.shape[-2], w.shape[-1]
    out = torch.empty_like(w, memory_format=torch.contiguous_format)
    moe_pack_weights(dtype, w.numel() // (rows * cols) if w.numel() else 0, rows, cols, w, out,
                     stream)
    return out


def make_profile(events) -> Profile:
    """Stage-boundary events (torch.cuda.Event or raw hipEvent_t ints, or
    None); a torch event is recorded once first so its handle exists."""
    handles = []
    for e in list(events) + [None] * (6 - len(events)):
        if e is None:
            handles.append(None)
        elif isinstance(e, int):
            handles.append(e)
        else:
            if not e.cuda_event:
                e.record()
            handles.append(e.cuda_event)
    return Profile((ctypes.c_void_p * 6)(*handles))


def moe_layer_forward_profiled(shape, weights: Weights, slot_map: SlotMap, T, h, out, ws,
                               profile: Profile, stream=None):
    _check("moe_layer_forward_profiled", lib().moe_layer_forward_profiled(
        ctypes.byref(shape), ctypes.byref(weights), ctypes.byref(slot_map), T, _p(h), _p(out),
        _p(ws), _nbytes(ws), ctypes.byref(profile), _stream(stream)))


def make_weights(*, w_router, bias=None, w_gate, w_up, w_down, sh_gate=None, sh_up=None,
                 sh_down=None) -> Weights:
    return Weights(*(_p(t) for t in (w_router, bias, w_gate, w_up, w_down, sh_gate, sh_up,
                                     sh_down)))


def make_slot_map(rep_off, rep_slot, seed: int) -> SlotMap:
    return SlotMap(_p(rep_off), _p(rep_slot), seed)


# ---------------------------------------------------------------- EPLB-lite

def moe_expert_counts(shape, T, topk_idx, counts, stream=None):
    _check("moe_expert_counts", lib().moe_expert_counts(
        ctypes.byref(shape), T, _p(topk_idx), _p(counts), _stream(stream)))


def make_eplb_config(*, n_experts, n_ranks, window, max_moves=2, spare_slots=1,
                     threshold=1.2) -> EplbConfig:
    return EplbConfig(n_experts, n_ranks, window, max_moves, spare_slots, threshold)


def _host(a, dtype):
    import numpy as np
    if not (isinstance(a, np.ndarray) and a.dtype == dtype and a.flags.c_contiguous):
        raise ValueError(f"expected a C-contiguous numpy {np.dtype(dtype).name} array")
    return a.ctypes.data


def moe_eplb_state_bytes(cfg: EplbConfig) -> int:
    return int(lib().moe_eplb_state_bytes(ctypes.byref(cfg)))


def moe_eplb_init(cfg: EplbConfig, state):
    """state: host numpy uint8 array of moe_eplb_state_bytes(cfg) bytes."""
    import numpy as np
    _check("moe_eplb_init", lib().moe_eplb_init(ctypes.byref(cfg), _host(state, np.uint8),
                                                state.nbytes))


def moe_eplb_observe(state, counts):
    import numpy as np
    _check("moe_eplb_observe", lib().moe_eplb_observe(_host(state, np.uint8),
                                                      _host(counts, np.int32)))


def moe_eplb_loads(state, n_ranks: int):
    import numpy as np
    loads = np.empty(n_ranks, np.float64)
    imb = ctypes.c_double()
    _check("moe_eplb_loads", lib().moe_eplb_loads(_host(state, np.uint8), _host(loads, np.float64),
                                                  ctypes.byref(imb)))
    return loads, imb.value


def moe_eplb_rebalance(state, max_moves: int):
    import numpy as np
    n = ctypes.c_int32()
    moves = np.zeros((max(max_moves, 1), 2), np.int32)
    _check("moe_eplb_rebalance", lib().moe_eplb_rebalance(_host(state, np.uint8),
                                                          ctypes.byref(n), _host(moves, np.int32)))
    return [tuple(int(v) for v in m) for m in moves[: n.value]]


def moe_eplb_slot_map(state, cfg: EplbConfig, rank: int):
    """(rep_off [E+1], rep_slot [nnz], slot_expert [S]) host arrays."""
    import numpy as np
    E, R, sp = cfg.n_experts, cfg.n_ranks, cfg.spare_slots
    off = np.empty(E + 1, np.int32)
    slot = np.empty(E + R * sp, np.int32)
    se = np.empty(E // R + sp, np.int32)
    n = ctypes.c_int32()
    _check("moe_eplb_slot_map", lib().moe_eplb_slot_map(
        _host(state, np.uint8), rank, _host(off, np.int32), _host(slot, np.int32),
        _host(se, np.int32), ctypes.byref(n)))
    return off, slot[: off[E]].copy(), se[: n.value].copy()


def moe_eplb_cleanup(state, cfg: EplbConfig):
    """Step 4 of section 6.2: reclaim the original-position copies of the
    migrations since the last cleanup; returns [(expert, rank, slot)]."""
    import numpy as np
    cap = cfg.n_experts * cfg.n_ranks
    out = np.zeros((cap, 3), np.int32)
    n = ctypes.c_int32()
    _check("moe_eplb_cleanup", lib().moe_eplb_cleanup(_host(state, np.uint8), cap,
                                                      ctypes.byref(n), _host(out, np.int32)))
    return [tuple(int(v) for v in r) for r in out[: n.value]]
