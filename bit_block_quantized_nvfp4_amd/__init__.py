"""NVFP4 routed-MoE FFN layer for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmoe_nvfp4.so`` (C ABI in
``include/moe_nvfp4.h``); ``ops`` is its thin Python binding.
"""
from .ops import (  # noqa: F401
    MOE_ACT_BF16,
    MOE_ACT_FP8_ROUTED,
    MOE_ACT_FP8_ROW,
    MOE_ACT_FP8_SHARED,
    NVFP4Router,
    NVFP4Weights,
    moe_combine,
    moe_combine_gated,
    moe_expert_ffn,
    moe_expert_ffn_combine,
    moe_expert_ffn_noalloc,
    moe_init,
    moe_layer,
    moe_permute,
    moe_route_permute,
    moe_route_topk,
    moe_router_topk,
    workspace_bytes,
)
