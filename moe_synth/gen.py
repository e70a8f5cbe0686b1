"""Workload definitions and seeded generators (no layer arithmetic here).

Workloads follow the DeepSeek-V3 layer shapes used throughout the expert
parallelism blog page (yveltals, section 2.1 and the Step 1-5 walk-through of
section 2.2): hidden 7168, 256 routed experts, top-8, SwiGLU intermediate 2048,
2 shared experts.

Distributions
-------------
* hidden states: N(0, 1), rounded to the compute dtype (fp16 RNE or fp32);
* router rows, shared-gate vector, expert matrices: fp16 workloads draw
  U(-sqrt(3/fan_in), +sqrt(3/fan_in)); the fp32 tiny workload draws
  N(0, 1)/sqrt(fan_in).  Either way each output of a projection of a
  unit-variance input has unit variance, so logits and pre-activations are
  ~N(0, 1);
* long-tail routing: 30% of the experts (77 of 256) get the same logit bias
  ``LONG_TAIL_BETA``; with unit-variance logits and top-8 this sends ~60% of
  the (token, expert) pairs to the hot 30% (the share quoted in section 6.1 of
  the blog page).  The hot ids are drawn from the seed.
"""
from __future__ import annotations

import collections
import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional

import numpy as np

# Sub-stream ids: one per tensor family.
_TID = {
    "hidden": 1,
    "router": 2,
    "shared_gate_vec": 3,
    "gate": 4,
    "up": 5,
    "down": 6,
    "sh_gate": 7,
    "sh_up": 8,
    "sh_down": 9,
    "hot": 10,
}

# Bias applied to the hot experts' logits.  Calibrated by Monte Carlo on
# unit-variance logits (256 experts, 77 hot, top-8): hot share 0.600.
LONG_TAIL_BETA = np.float32(0.57)
HOT_FRACTION = 0.3


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens in the batch
    H: int                 # hidden size
    I: int                 # SwiGLU intermediate size
    E: int                 # routed (logical) experts
    K: int                 # experts per token
    n_shared: int          # shared experts (0 = partial rank-share output)
    dtype: str             # "f32" or "f16": activations and weights
    dispatch: str          # "same" or "fp8"
    ep_size: int           # 1 = full layer resident on this GPU
    ep_rank: int           # which rank's share this GPU computes
    replica: bool          # one redundant replica of a hot remote expert
    long_tail: bool        # per-expert logit bias
    seed: int
    prompts: int = 1       # prefill batches: T = prompts * tokens per prompt
    n_groups: int = 0      # group-limited routing: expert groups (0 = off)
    topk_groups: int = 0   # groups kept per token

    @property
    def groups(self):
        return (self.n_groups, self.topk_groups) if self.n_groups else None

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.float16

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _cfg(**kw) -> MoEConfig:
    return MoEConfig(**kw)


# The five workloads of the build, numbered 1..5.
CONFIGS = {
    1: _cfg(name="tiny_fp32_T64", T=64, H=256, I=128, E=16, K=2, n_shared=1,
            dtype="f32", dispatch="same", ep_size=1, ep_rank=0, replica=False,
            long_tail=False, seed=1),
    2: _cfg(name="ep8_rank0_decode_T256", T=256, H=7168, I=2048, E=256, K=8,
            n_shared=0, dtype="f16", dispatch="same", ep_size=8, ep_rank=0,
            replica=False, long_tail=False, seed=2),
    3: _cfg(name="full_layer_decode_T128", T=128, H=7168, I=2048, E=256, K=8,
            n_shared=2, dtype="f16", dispatch="same", ep_size=1, ep_rank=0,
            replica=False, long_tail=True, seed=3),
    4: _cfg(name="ep8_rank0_prefill_T16384", T=16384, H=7168, I=2048, E=256,
            K=8, n_shared=0, dtype="f16", dispatch="same", ep_size=8,
            ep_rank=0, replica=False, long_tail=False, seed=4, prompts=16),
    5: _cfg(name="ep8_rank0_replica_fp8_T512", T=512, H=7168, I=2048, E=256,
            K=8, n_shared=0, dtype="f16", dispatch="fp8", ep_size=8, ep_rank=0,
            replica=True, long_tail=True, seed=5),
}


def config(n: int, seed: Optional[int] = None, **overrides) -> MoEConfig:
    c = CONFIGS[n]
    if seed is not None:
        overrides["seed"] = seed
    return dataclasses.replace(c, **overrides) if overrides else c


def scaled_config(n: int, *, T: int, H: int, I: int, seed: Optional[int] = None,
                  **overrides) -> MoEConfig:
    """Same routing structure as workload ``n`` with smaller dense dims."""
    return config(n, seed=seed, T=T, H=H, I=I, **overrides)


def _rng(seed: int, tensor: str, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, _TID[tensor], expert])))


def _weights(cfg: MoEConfig, rng: np.random.Generator, shape, fan_in: int):
    n = int(np.prod(shape))
    if cfg.dtype == "f32":
        w = rng.standard_normal(n, dtype=np.float32) * np.float32(1.0 / np.sqrt(fan_in))
        return w.reshape(shape)
    a = np.float32(np.sqrt(3.0 / fan_in))
    w = rng.random(n, dtype=np.float32) * (2 * a) - a
    return w.astype(np.float16).reshape(shape)


def gen_hidden(cfg: MoEConfig, T: Optional[int] = None) -> np.ndarray:
    """Hidden states [T, H], N(0, 1) in the compute dtype."""
    T = cfg.T if T is None else T
    x = _rng(cfg.seed, "hidden").standard_normal(T * cfg.H, dtype=np.float32)
    return x.astype(cfg.np_dtype).reshape(T, cfg.H)


def gen_router(cfg: MoEConfig) -> np.ndarray:
    """Router rows [E, H] (row e scores expert e; the transpose of the
    page's [hidden, experts] math shape) plus, when the layer has shared
    experts, one extra row [H] for the shared-expert gate vector.

    Returns an array [E + (n_shared > 0), H].
    """
    w = _weights(cfg, _rng(cfg.seed, "router"), (cfg.E, cfg.H), cfg.H)
    if cfg.n_shared:
        g = _weights(cfg, _rng(cfg.seed, "shared_gate_vec"), (1, cfg.H), cfg.H)
        w = np.concatenate([w, g], axis=0)
    return np.ascontiguousarray(w)


def gen_hot_experts(cfg: MoEConfig) -> np.ndarray:
    """Sorted ids of the hot experts (30% of E), drawn from the seed."""
    n_hot = int(round(HOT_FRACTION * cfg.E))
    ids = _rng(cfg.seed, "hot").choice(cfg.E, n_hot, replace=False)
    return np.sort(ids).astype(np.int32)


def gen_router_bias(cfg: MoEConfig) -> Optional[np.ndarray]:
    """fp32 bias [E] (LONG_TAIL_BETA on hot experts, 0 elsewhere) or None."""
    if not cfg.long_tail:
        return None
    b = np.zeros(cfg.E, dtype=np.float32)
    b[gen_hot_experts(cfg)] = LONG_TAIL_BETA
    return b


def replica_expert(cfg: MoEConfig) -> Optional[int]:
    """The expert that gets one redundant replica on this GPU: the lowest-id
    hot expert that is owned by another rank (id >= E/ep_size for rank 0)."""
    if not cfg.replica:
        return None
    per = cfg.E // cfg.ep_size
    lo, hi = cfg.ep_rank * per, (cfg.ep_rank + 1) * per
    for e in gen_hot_experts(cfg):
        if not (lo <= e < hi):
            return int(e)
    raise ValueError("no remote hot expert")


def gen_expert(cfg: MoEConfig, e: int):
    """Routed expert ``e``: (gate [I,H], up [I,H], down [H,I]), out-major."""
    g = _weights(cfg, _rng(cfg.seed, "gate", e), (cfg.I, cfg.H), cfg.H)
    u = _weights(cfg, _rng(cfg.seed, "up", e), (cfg.I, cfg.H), cfg.H)
    d = _weights(cfg, _rng(cfg.seed, "down", e), (cfg.H, cfg.I), cfg.I)
    return g, u, d


def gen_shared_expert(cfg: MoEConfig, j: int):
    """Shared expert ``j``: (gate [I,H], up [I,H], down [H,I]), out-major."""
    g = _weights(cfg, _rng(cfg.seed, "sh_gate", j), (cfg.I, cfg.H), cfg.H)
    u = _weights(cfg, _rng(cfg.seed, "sh_up", j), (cfg.I, cfg.H), cfg.H)
    d = _weights(cfg, _rng(cfg.seed, "sh_down", j), (cfg.H, cfg.I), cfg.I)
    return g, u, d


def gen_slot_weights(cfg: MoEConfig, slot_experts):
    """Stacked weights for local slots holding the given logical experts:
    (gate [S,I,H], up [S,I,H], down [S,H,I])."""
    S = len(slot_experts)
    G = np.empty((S, cfg.I, cfg.H), cfg.np_dtype)
    U = np.empty((S, cfg.I, cfg.H), cfg.np_dtype)
    D = np.empty((S, cfg.H, cfg.I), cfg.np_dtype)
    for s, e in enumerate(slot_experts):
        G[s], U[s], D[s] = gen_expert(cfg, int(e))
    return G, U, D


def gen_shared_weights(cfg: MoEConfig):
    """Stacked shared-expert weights, or (None, None, None)."""
    if not cfg.n_shared:
        return None, None, None
    parts = [gen_shared_expert(cfg, j) for j in range(cfg.n_shared)]
    return tuple(np.ascontiguousarray(np.stack(p)) for p in zip(*parts))


def iter_experts(cfg: MoEConfig, experts: Iterable[int], workers: Optional[int] = None):
    """Yield (e, (gate, up, down)) for ``experts`` in order, drawn on a
    thread pool (numpy releases the GIL while drawing) with a bounded
    look-ahead so at most ~2*workers experts are held at once."""
    workers = workers or min(16, os.cpu_count() or 1)
    it = iter(int(e) for e in experts)
    with ThreadPoolExecutor(workers) as ex:
        pending = collections.deque()
        for _ in range(2 * workers):
            e = next(it, None)
            if e is None:
                break
            pending.append((e, ex.submit(gen_expert, cfg, e)))
        while pending:
            e, fut = pending.popleft()
            yield e, fut.result()
            nxt = next(it, None)
            if nxt is not None:
                pending.append((nxt, ex.submit(gen_expert, cfg, nxt)))
