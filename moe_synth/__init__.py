"""Seeded synthetic inputs for the MoE-layer hot path.

This module only draws numbers: hidden states, weights, router bias and the
deployment choices of each workload (which rank of an EP group this GPU plays,
which expert gets a redundant replica).  It holds none of the layer's
arithmetic (no routing, no softmax, no dispatch, no expert math), so both the
HIP path and the CPU oracle may consume its outputs.

Every tensor comes from its own ``SeedSequence([seed, tensor_id, expert])``
sub-stream, so one expert's weights can be regenerated without the others.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    MoEConfig,
    config,
    gen_hidden,
    gen_router,
    gen_router_bias,
    gen_hot_experts,
    gen_expert,
    gen_shared_expert,
    gen_slot_weights,
    iter_experts,
    gen_shared_weights,
    replica_expert,
    LONG_TAIL_BETA,
    scaled_config,
)
