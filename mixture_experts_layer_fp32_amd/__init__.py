"""MoE layer forward (one GPU's share) for AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels inside libmoe.so, reached
through its C ABI (include/moe.h, include/moe_mxfp8.h, include/moe_backward.h,
include/moe_variants.h). This package is the thin Python binding
(same function names as the C entry points) plus owners of device buffers.
Importing it does not load the library; the first call does, and it raises
if libmoe.so has not been built (there is no fallback implementation).
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, MOE_BF16, MOE_F32, MOE_MAX_EXPERTS, MOE_MAX_TOPK, MoeError, load_library,
    make_desc, moe_desc, moe_expert_down, moe_expert_ffn, moe_expert_gate_up,
    moe_ffn_workspace_size, moe_layer_forward, moe_permute, moe_permute_workspace_size, moe_route,
    moe_unpermute_combine, moe_workspace_size, workspace,
    moe_mxfp8_quantize_rows, moe_mxfp8_pack_weights, moe_expert_ffn_mxfp8,
    moe_ffn_mxfp8_workspace_size, moe_expert_gate_up_mxfp8, moe_expert_down_mxfp8,
    moe_expert_ffn_train, moe_combine_backward, moe_expert_ffn_backward,
    moe_ffn_backward_workspace_size,
    moe_router_backward, moe_router_backward_workspace_size, moe_input_backward,
    moe_layer_backward, moe_backward_workspace_size, moe_expert_gate_up_backward,
    moe_expert_weight_grad, moe_route_typed, MOE_F16, moe_expert_ffn_ptrs, pointer_array,
    moe_ffn_tile_shape, moe_pack_expert_weights, pack_expert_weights, MOE_WEIGHTS_PACKED,
    MOE_WEIGHTS_STACKED, moe_permute_noalloc, moe_down_workspace_size, moe_gate_up_workspace_size,
    moe_route_workspace_size,
)
from .layer import EPRankShareForward, LayerForward, LayerForwardMXFP8, LayerTrain  # noqa: F401
