/*
 * MXFP8 variant of the grouped expert FFN (libmoe, AMD MI355X / gfx950).
 *
 * The pages name an MXFP8 transform of the MoE layer (torchtitan issue 5554:
 * the shared-expert overlap covers the layer's BF16 and MXFP8 transforms)
 * without defining the format. Format used here: OCP Microscaling (MX) v1.0,
 * MXFP8 with E4M3 elements -- one E8M0 scale byte 2^(s) (stored s + 127) per
 * 32 consecutive values along the contraction dimension K, with
 * s = floor(log2(max |v|)) - 8 clamped to [-127, 127] (all-zero block:
 * byte 0), elements v / 2^s rounded to the nearest E4M3 value (ties to even)
 * and saturated at +-448.
 *
 * Layouts (all DEVICE memory, caller-owned; the library allocates nothing):
 *   activation rows  codes [rows, K] uint8, scales [rows, K / 32] uint8
 *   packed weights   codes [n, N, K] uint8, scales [n, N, K / 32] uint8 --
 *                    output column c of expert e holds its K values
 *                    contiguously (quantized along K, per column)
 * Every call enqueues on `stream` and returns without synchronising; errors
 * are returned as moe_status codes (moe_status_str), checked on the host
 * before any HIP call.
 */
#ifndef MOE_MXFP8_H
#define MOE_MXFP8_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_mxfp8_quantize_rows - quantize bf16 rows along K.
 * (OCP MX v1.0 as above; used for the activations entering the expert GEMMs.)
 *
 *  rows    number of rows (>= 0; 0 does nothing)
 *  K       row length, a positive multiple of 32
 *  x       [rows, K] bf16
 *  codes   [rows, K] uint8 out
 *  scales  [rows, K / 32] uint8 out
 * Errors: INVALID_ARG (negative rows, K not a positive multiple of 32, NULL
 * buffer with rows > 0), UNSUPPORTED (rows * K >= 2^40).
 */
moe_status moe_mxfp8_quantize_rows(int64_t rows, int32_t K, const void* x, void* codes,
                                   void* scales, void* stream);

/*
 * moe_mxfp8_pack_weights - quantize stacked expert weights per output column
 * along K and store them K-contiguous (the layout moe_expert_ffn_mxfp8
 * reads). Page "Expert Parallel (EP)", Requirements (tensor-style stacked
 * gate_up_proj [n, D, 2I] and down_proj [n, I, D]). Meant to run once, when
 * the weights are loaded.
 *
 *  n       experts (>= 0)
 *  K, N    w is [n, K, N]; K a positive multiple of 32, N > 0
 *  w       [n, K, N] bf16
 *  codes   [n, N, K] uint8 out
 *  scales  [n, N, K / 32] uint8 out
 * Errors: INVALID_ARG (bad sizes, NULL buffer with n > 0),
 * UNSUPPORTED (n * K * N >= 2^40).
 */
moe_status moe_mxfp8_pack_weights(int32_t n, int32_t K, int32_t N, const void* w, void* codes,
                                  void* scales, void* stream);

/*
 * moe_expert_ffn_mxfp8 - moe_expert_ffn in MXFP8: every local expert's
 * SiLU-gated two-layer FFN on its segment of rows (page "Expert Parallel
 * (EP)", Communication Pattern stage 3; page "Worked Example", Step 3), with
 * both GEMMs on the block-scaled FP8 matrix instructions and fp32
 * accumulation. H = SiLU(G) * U is formed in fp32, rounded to bf16, then
 * quantized along I for the down projection; Y is fp32.
 *
 *  desc        a bf16 layer (act_dtype MOE_BF16); D and inter multiples of 128
 *  n_experts   local experts (1 .. MOE_MAX_EXPERTS)
 *  inter       intermediate size I
 *  cap_rows    rows of the activation codes / y_perm
 *  xq, xs      activation codes [cap_rows, D], scales [cap_rows, D / 32]
 *  offsets     [n_experts + 1] int32 DEVICE: expert j owns rows
 *              [offsets[j], offsets[j+1])
 *  w_gu_q, w_gu_s  packed gate_up_proj: codes [n, 2 inter, D], scales
 *              [n, 2 inter, D / 32] (moe_mxfp8_pack_weights of [n, D, 2I])
 *  w_d_q, w_d_s    packed down_proj: codes [n, D, inter], scales
 *              [n, D, inter / 32] (moe_mxfp8_pack_weights of [n, I, D])
 *  y_perm      [cap_rows, D] fp32 out (rows past offsets[n] untouched)
 *  ws          workspace of at least moe_ffn_mxfp8_workspace_size() bytes
 *              (H in bf16, then its codes and scales)
 * Errors: as moe_expert_ffn; UNSUPPORTED for a non-bf16 layer or D, inter not
 * multiples of 128.
 */
moe_status moe_expert_ffn_mxfp8(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                int64_t cap_rows, const void* xq, const void* xs,
                                const int32_t* offsets, const void* w_gu_q, const void* w_gu_s,
                                const void* w_d_q, const void* w_d_s, float* y_perm, void* ws,
                                size_t ws_bytes, void* stream);
size_t moe_ffn_mxfp8_workspace_size(const moe_desc* desc, int32_t inter, int64_t cap_rows);

/*
 * The halves of moe_expert_ffn_mxfp8, for callers that keep H themselves
 * (page "Worked Example", Step 3: first and second layer of the expert FFN).
 * moe_expert_gate_up_mxfp8: h[r, c] = bf16(SiLU(x[r] . W_gate[c]) * (x[r] . W_up[c]))
 *   from the MXFP8 activations and packed gate_up_proj; h is [cap_rows, inter]
 *   bf16 (rows past offsets[n] untouched).
 * moe_expert_down_mxfp8: y_perm = h . W_down from H's MXFP8 codes hq
 *   [cap_rows, inter] and scales hs [cap_rows, inter / 32] (e.g. from
 *   moe_mxfp8_quantize_rows of h) and the packed down_proj; y_perm fp32.
 * Other arguments and errors as for moe_expert_ffn_mxfp8.
 */
moe_status moe_expert_gate_up_mxfp8(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                    int64_t cap_rows, const void* xq, const void* xs,
                                    const int32_t* offsets, const void* w_gu_q,
                                    const void* w_gu_s, void* h, void* stream);
moe_status moe_expert_down_mxfp8(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                 int64_t cap_rows, const void* hq, const void* hs,
                                 const int32_t* offsets, const void* w_d_q, const void* w_d_s,
                                 float* y_perm, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP8_H */
