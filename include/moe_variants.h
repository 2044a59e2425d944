/*
 * Interface variants of the MoE layer forward (libmoe, AMD MI355X / gfx950):
 * the router in a 16-bit router dtype, and experts held as separate
 * per-expert weight buffers.
 *
 * Page "Expert Parallel (EP)", Configuration: router_dtype is 'fp32', 'bf16'
 * or 'fp16'; Requirements: experts are either an nn.ModuleList (one module,
 * hence one weight buffer, per expert) or tensor-style stacked
 * gate_up_proj / down_proj, and both are supported.
 *
 * Conventions as in moe.h: caller-owned DEVICE memory, work enqueued on
 * `stream`, host-side argument checks before any HIP call, moe_status codes.
 */
#ifndef MOE_VARIANTS_H
#define MOE_VARIANTS_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_route_typed - moe_route with the router in router_dtype (MOE_F32,
 * MOE_BF16 or MOE_F16). The gate weight is held in router_dtype; each logit
 * is the token . weight-row dot product (exact products, fp64 sum) rounded
 * once to nearest even to router_dtype; a bias is added to that value and
 * the sum rounded again to router_dtype. Softmax and top-k (ties to the lower
 * expert id) then run on those logits in fp32, as in moe_route. MOE_F32
 * makes moe_route's choices with every logit the reference logit (no
 * workspace; the fp64 matrix cores compute all of them).
 *
 *  router_dtype  MOE_F32, MOE_BF16 or MOE_F16
 *  x          [T, D] act
 *  w_router   [E, D] router_dtype
 *  logit_bias [E] fp32 | NULL
 *  logits     [T, E] router_dtype | NULL  out
 *  probs      [T, E] fp32 | NULL          out: softmax over all E logits
 *  topk_idx   [T, top_k] int32, topk_w [T, top_k] fp32  out
 * Errors: as moe_route; INVALID_ARG for another router_dtype.
 */
moe_status moe_route_typed(const moe_desc* desc, int32_t router_dtype, const void* x,
                           const void* w_router, const float* logit_bias, void* logits,
                           float* probs, int32_t* topk_idx, float* topk_w, void* stream);

/*
 * moe_expert_ffn_ptrs - moe_expert_ffn with ModuleList-style experts: each
 * local expert's weights are buffers of their own, found through device
 * arrays of pointers (same per-expert layouts as the stacked tensors).
 *
 *  w_gate_up_ptrs  [n_experts] DEVICE array of pointers, entry j to expert
 *                  j's gate_up_proj [D, 2 inter] bf16
 *  w_down_ptrs     [n_experts] DEVICE array of pointers, entry j to expert
 *                  j's down_proj [inter, D] bf16
 * Other arguments, the workspace (moe_ffn_workspace_size) and the results as
 * for moe_expert_ffn; bf16 layers only (UNSUPPORTED for fp32 layers).
 */
moe_status moe_expert_ffn_ptrs(const moe_desc* desc, int32_t n_experts, int32_t inter,
                               int64_t cap_rows, const void* x_perm, const int32_t* offsets,
                               const void* const* w_gate_up_ptrs,
                               const void* const* w_down_ptrs, void* y_perm, void* ws,
                               size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_VARIANTS_H */
