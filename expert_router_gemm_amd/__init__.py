"""MI355X-native MoE-layer hot path: router + top-K, dispatch, SwiGLU grouped
GEMM, combine (libmoe, HIP for gfx950) and its Python binding."""
from .binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MOE_F16,
    MOE_F32,
    MOE_F_SHARED,
    MOE_FP8_E4M3,
    MoEError,
    Shape,
    SlotMap,
    Weights,
    lib,
    make_shape,
    make_slot_map,
    make_weights,
    moe_combine,
    moe_dispatch,
    moe_expert_ffn,
    moe_expert_ffn_down,
    moe_expert_ffn_up,
    moe_layer_forward,
    moe_route,
    moe_workspace_bytes,
    status_str,
    version,
)
from .placement import build_slot_map, contiguous_owner, drop_replica  # noqa: F401
