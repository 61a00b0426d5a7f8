"""MI355X-native MoE expert-parallel layer: route, dispatch, grouped SwiGLU FFN, combine.

The compute runs in libmoe_route.so (HIP kernels for gfx950, C ABI in
include/moe_route.h); ``binding`` marshals torch tensors into its calls.
"""
from .binding import (  # noqa: F401
    MoeError,
    MoeLayer,
    PackedFfnWeights,
    alloc_route_plan,
    load_library,
    moe_abi_version,
    moe_capacity,
    moe_combine,
    moe_combine_fp8,
    moe_dispatch,
    moe_dispatch_fp8,
    moe_dispatch_planned,
    moe_dispatch_workspace_bytes,
    moe_exchange_plan,
    moe_exchange_workspace_bytes,
    moe_fp8_dequantize_rows,
    moe_fp8_quantize_rows,
    moe_grouped_ffn,
    moe_grouped_ffn_packed,
    moe_grouped_ffn_workspace_bytes,
    moe_pack_ffn_weights,
    moe_packed_ffn_weight_bytes,
    moe_reroute_overflow,
    moe_reroute_workspace_bytes,
    moe_route_plan,
    moe_route_plan_bytes,
    moe_route_topk,
    moe_router_logits,
    moe_rows_permute,
)
