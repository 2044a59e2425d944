/*
 * Backward pass of the MoE layer (libmoe, AMD MI355X / gfx950).
 *
 * The pages describe expert parallelism as training middleware (page "Expert
 * Parallel (EP)", Overview) and define the forward (Communication Pattern,
 * stages 1-4; page "Worked Example", Steps 1-5). These calls compute the
 * exact gradients of that forward, with the readings:
 *  - the top-k choice is piecewise constant: gradients flow through the
 *    routing weights of the chosen experts only (renormalised top-k weights,
 *    norm_topk = 1, are the softmax over the chosen logits);
 *  - the input gradient adds (shared + routed) + router contributions in that
 *    order, then the residual's (torchtitan issue 5554: the input fork keeps
 *    the original order of the three contributions);
 *  - the permuted rows x_perm and the expert outputs y_perm of the forward
 *    are inputs (twinkle pull request 198: the forward returns the permuted
 *    tokens so the backward path keeps them).
 * Precision, bf16 layers: bf16 operands on the matrix cores with fp32
 * accumulation; the gate and up pre-activations G | U are used in fp32 (never
 * rounded: the SiLU derivative would turn a bf16 G's rounding into errors of
 * dG well above dG's own rounding), either saved by the training forward
 * (moe_expert_ffn_train) or recomputed from x_perm; dH is fp32; dy_perm,
 * dG | dU and H are bf16; every weight gradient and dx_perm are fp32; dx is
 * rounded once to bf16. Saved and recomputed G | U are the same bits (the
 * same products in the same order), so both give the same gradients, bit for
 * bit. fp32 layers: fp32 throughout (vector ALUs), G | U always recomputed,
 * with "bf16" below read as fp32 for dout, dy_perm, x_perm, dG | dU, H and
 * dx.
 *
 * Conventions as in moe.h: caller-owned DEVICE memory, work enqueued on
 * `stream`, host-side argument checks before any HIP call, moe_status codes.
 * Every call returns MOE_ERR_UNSUPPORTED for norm_topk = 0 (plain top-k
 * weights).
 */
#ifndef MOE_BACKWARD_H
#define MOE_BACKWARD_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_combine_backward - adjoint of moe_unpermute_combine and of the routing
 * weights (page "Expert Parallel (EP)", Communication Pattern stage 4; page
 * "Worked Example", Steps 1 and 4). For every token t and slot j with
 * p = pos[t,j] >= 0:
 *   dtopk_w[t,j] = dout[t] . y_perm[p]            (fp32 dot)
 *   dy_perm[p]   = bf16(topk_w[t,j] * dout[t])
 *   dlogit[t,j]  = topk_w[t,j] * (dtopk_w[t,j] - sum_i topk_w[t,i] dtopk_w[t,i])
 *                  (gradient of the logit of expert topk_idx[t,j]; slots with
 *                  pos < 0 count as dtopk_w = 0, so the value is the layer's
 *                  gradient only when every slot's expert is local)
 *   dl_perm[p]   = dlogit[t,j]
 *
 *  dout     [T, D] bf16          gradient of the layer output
 *  y_perm   [rows, D] fp32       expert outputs of the forward
 *  pos      [T, top_k] int32, topk_w [T, top_k] fp32   (forward routing)
 *  dy_perm  [rows, D] bf16 out   (rows not named by pos untouched)
 *  dtopk_w  [T, top_k] fp32 out | NULL
 *  dlogit   [T, top_k] fp32 out
 *  dl_perm  [rows] fp32 out | NULL
 * Errors: INVALID_ARG (NULL required pointer), UNSUPPORTED (see above).
 */
moe_status moe_combine_backward(const moe_desc* desc, const void* dout, const float* y_perm,
                                const int32_t* pos, const float* topk_w, void* dy_perm,
                                float* dtopk_w, float* dlogit, float* dl_perm, void* stream);

/*
 * moe_expert_ffn_train - moe_expert_ffn for a training step (bf16 layers):
 * the same y_perm, bit for bit, and the gate and up pre-activations kept for
 * the backward (page "Expert Parallel (EP)", Communication Pattern stage 3:
 * the expert FFN, whose backward needs G and U).
 *
 *  arguments as for moe_expert_ffn, and
 *  gu_saved [cap_rows, 2 inter] fp32 out   G | U = x_perm[r] Wgu_e for the
 *           rows r of each expert segment (rows past offsets[n] untouched);
 *           hand it to moe_expert_ffn_backward / moe_layer_backward, which
 *           then skip the recompute of G | U and the round trip of dH through
 *           memory (cap_rows * 2 inter * 4 bytes of HBM held from the
 *           forward to the backward).
 * Errors: as moe_expert_ffn; UNSUPPORTED for fp32 layers; INVALID_ARG for
 * offsets NULL with n_experts != 1.
 */
moe_status moe_expert_ffn_train(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                int64_t cap_rows, const void* x_perm, const int32_t* offsets,
                                const void* w_gate_up, const void* w_down, void* y_perm,
                                float* gu_saved, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn_backward - gradients of moe_expert_ffn (page "Expert
 * Parallel (EP)", Communication Pattern stage 3 and Requirements; page
 * "Worked Example", Step 3). Per expert segment, with G | U = X Wgu
 * (saved or recomputed), s = sigmoid(G), H = G s U:
 *   dH  = dY Wd^T
 *   dG  = dH U (s + G s (1 - s)),  dU = dH G s
 *   dX  = [dG | dU] Wgu^T,  dWd = H^T dY,  dWgu = X^T [dG | dU]
 *
 *  n_experts, inter, cap_rows, x_perm, offsets, w_gate_up, w_down
 *             as for moe_expert_ffn (offsets NULL: one expert owning all rows)
 *  dy_perm    [cap_rows, D] bf16   gradient of y_perm
 *  gu_saved   [cap_rows, 2 inter] fp32 | NULL: G | U from moe_expert_ffn_train
 *             on the same x_perm, offsets and w_gate_up (NULL: recomputed;
 *             non-NULL with an fp32 layer: UNSUPPORTED)
 *  dx_perm    [cap_rows, D] fp32 out | NULL (rows past offsets[n] untouched)
 *  dw_gate_up [n_experts, D, 2 inter] fp32 out (every expert written: zero
 *             for an expert without rows)
 *  dw_down    [n_experts, inter, D] fp32 out (likewise)
 *  ws         workspace of at least moe_ffn_backward_workspace_size() bytes
 *             (dH in fp32, dG | dU and H in bf16; dH unused with gu_saved)
 * Errors: as moe_expert_ffn; UNSUPPORTED also when cap_rows * max(D, 2 inter)
 * * 2 bytes reaches 2^30.
 */
moe_status moe_expert_ffn_backward(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                   int64_t cap_rows, const void* x_perm, const int32_t* offsets,
                                   const void* w_gate_up, const void* w_down,
                                   const void* dy_perm, const float* gu_saved, float* dx_perm,
                                   float* dw_gate_up, float* dw_down, void* ws, size_t ws_bytes,
                                   void* stream);
size_t moe_ffn_backward_workspace_size(const moe_desc* desc, int32_t inter, int64_t cap_rows);

/*
 * The pieces of moe_expert_ffn_backward, for callers that schedule them
 * apart (for instance weight gradients after the input gradients).
 *
 * moe_expert_gate_up_backward - adjoint of the gated first layer given
 *   dH [cap_rows, inter] fp32 (= dY W_down^T): recomputes G | U = X Wgu per
 *   expert segment in fp32 and writes dgu = dG | dU [cap_rows, 2 inter] and
 *   h = SiLU(G) U [cap_rows, inter] (bf16; rows past offsets[n] untouched).
 *   Arguments otherwise as for moe_expert_ffn_backward.
 *
 * moe_expert_weight_grad - grouped weight-gradient GEMM: for each expert e,
 *   c[e] = a_e^T b_e (fp32 [P, Q]) where a_e, b_e are rows
 *   [offsets[e], offsets[e+1]) of a [cap_rows, P] and b [cap_rows, Q] (bf16);
 *   c[e] = 0 for an expert without rows. dW_down = H^T dY (a = h, P = inter,
 *   b = dy_perm, Q = D) and dW_gate_up = X^T [dG | dU] (a = x_perm, P = D,
 *   b = dgu, Q = 2 inter). P and Q are multiples of 64, at most 2^24.
 * Errors: as moe_expert_ffn_backward (UNSUPPORTED when cap_rows * max(P, Q)
 * * 2 bytes reaches 2^30, or P or Q exceeds 2^24).
 */
moe_status moe_expert_gate_up_backward(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                       int64_t cap_rows, const void* x_perm,
                                       const int32_t* offsets, const void* w_gate_up,
                                       const float* dh, void* dgu, void* h, void* stream);
moe_status moe_expert_weight_grad(const moe_desc* desc, int32_t n_experts, int64_t cap_rows,
                                  const void* a, int32_t P, const void* b, int32_t Q,
                                  const int32_t* offsets, float* c, void* stream);

/*
 * moe_router_backward - gradient of the router weight (page "[Question] How
 * does the gate coordinate across ranks in expert parallelism?": the gate
 * weight [num_experts, embedding_dim]; page "Worked Example", Step 1):
 *   dw_router[e] = sum over the permuted rows p of expert e of dl_perm[p] x_perm[p]
 * (= sum over tokens t choosing e of dlogit x[t]), in a fixed order (no
 * atomics: the result is the same on every run); 0 for an expert without rows.
 *
 *  cap_rows   rows of x_perm / dl_perm
 *  x_perm     [cap_rows, D] bf16
 *  offsets    [E + 1] int32 DEVICE: the permute over all E experts
 *  dl_perm    [cap_rows] fp32 (from moe_combine_backward)
 *  dw_router  [E, D] fp32 out
 *  ws         workspace of at least moe_router_backward_workspace_size() bytes
 */
moe_status moe_router_backward(const moe_desc* desc, int64_t cap_rows, const void* x_perm,
                               const int32_t* offsets, const float* dl_perm, float* dw_router,
                               void* ws, size_t ws_bytes, void* stream);
size_t moe_router_backward_workspace_size(const moe_desc* desc, int64_t cap_rows);

/*
 * moe_input_backward - the input gradient, summed in fp32 in the order of
 * torchtitan issue 5554 and rounded once:
 *   dx[t] = bf16(((dx_shared[t] + sum_j dx_perm[pos[t,j]])
 *                 + sum_j dlogit[t,j] w_router[topk_idx[t,j]]) + dout[t])
 * Slots with pos < 0 add no routed term; a NULL dx_shared, dlogit or dout
 * drops that term.
 *
 *  dx_perm [rows, D] fp32; pos, topk_idx [T, top_k] int32; dlogit [T, top_k]
 *  fp32 | NULL; w_router [E, D] fp32; dx_shared [T, D] fp32 | NULL;
 *  dout [T, D] bf16 | NULL; dx [T, D] bf16 out
 */
moe_status moe_input_backward(const moe_desc* desc, const float* dx_perm, const int32_t* pos,
                              const int32_t* topk_idx, const float* dlogit,
                              const float* w_router, const float* dx_shared, const void* dout,
                              void* dx, void* stream);

/*
 * moe_layer_backward - the whole layer's backward on this GPU (every expert
 * local, as moe_layer_forward): combine adjoint, expert FFN backward, shared
 * expert backward (I_shared > 0), router weight gradient, input gradient.
 *
 *  forward inputs: x [T, D] bf16, w_router [E, D] fp32, w_gate_up
 *    [E, D, 2I], w_down [E, I, D], shared_gate_up [D, 2 I_shared] | NULL,
 *    shared_down [I_shared, D] | NULL (bf16)
 *  forward results: topk_idx, topk_w [T, top_k]; offsets [E + 1] (device);
 *    pos [T, top_k]; x_perm [T top_k, D] bf16; y_perm [T top_k, D] fp32;
 *    gu_saved [T top_k, 2I] fp32 | NULL and gu_shared_saved
 *    [T, 2 I_shared] fp32 | NULL: G | U of the routed and the shared experts
 *    from moe_expert_ffn_train (NULL: recomputed; bf16 layers only)
 *  dout [T, D] bf16      gradient of the layer output
 *  dx [T, D] bf16 out; dw_router [E, D], dw_gate_up [E, D, 2I],
 *  dw_down [E, I, D] fp32 out; dw_shared_gate_up [D, 2 I_shared],
 *  dw_shared_down [I_shared, D] fp32 out (required when I_shared > 0)
 *  ws   workspace of at least moe_backward_workspace_size() bytes
 */
moe_status moe_layer_backward(const moe_desc* desc, const void* x, const float* w_router,
                              const void* w_gate_up, const void* w_down,
                              const void* shared_gate_up, const void* shared_down,
                              const int32_t* topk_idx, const float* topk_w,
                              const int32_t* offsets, const int32_t* pos, const void* x_perm,
                              const float* y_perm, const float* gu_saved,
                              const float* gu_shared_saved, const void* dout, void* dx,
                              float* dw_router,
                              float* dw_gate_up, float* dw_down, float* dw_shared_gate_up,
                              float* dw_shared_down, void* ws, size_t ws_bytes, void* stream);
size_t moe_backward_workspace_size(const moe_desc* desc);

#ifdef __cplusplus
}
#endif

#endif /* MOE_BACKWARD_H */
