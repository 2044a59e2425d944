/*
 * moe.h - C ABI of a Mixture-of-Experts layer forward for AMD MI355X (gfx950),
 * covering the work one GPU (one expert-parallel rank) does.
 *
 * The calls follow the four-stage expert-parallel forward described on the
 * page "Expert Parallel (EP)" (section Communication Pattern): preprocess
 * (per-expert counts and split sizes), permute tokens by expert, expert
 * compute, unpermute with routing weights; preceded by the router of
 * "Worked Example: Tracing a Token Through Expert Parallelism" (Step 1).
 * The all-to-all exchanges between ranks are not part of this library.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every data pointer is DEVICE memory owned by the caller (inputs, outputs,
 *    index maps, workspace). The library never allocates or frees memory and
 *    keeps no pointer after a call returns.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and the call returns without waiting. Results are ready once the
 *    caller synchronises the stream or waits on an event recorded after it.
 *    No call copies data to the host or synchronises.
 *  - Row-major layouts throughout. "act" arrays hold the activation dtype of
 *    the descriptor (fp32, or bf16 as raw 16-bit words); the router weight,
 *    logits, probabilities and routing weights are always fp32; indices are
 *    int32.
 *  - Argument checks run on the host before any HIP call, so a rejected call
 *    touches no device state and needs no GPU. With T == 0 (or cap_rows == 0
 *    for moe_expert_ffn) a call returns MOE_OK after checking the descriptor;
 *    moe_permute and moe_layer_forward then only write zero counts, offsets
 *    and split sizes, the other calls do nothing.
 *  - Status: MOE_OK, or one of the negative codes below. MOE_ERR_HIP means a
 *    kernel launch failed; moe_last_hip_error() returns the hipError_t.
 *    Calls on the same stream are ordered; calls that share outputs or
 *    workspace on different streams race.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* bad dimension, null required pointer, bad range */
  MOE_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels handle      */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than the *_workspace_size    */
  MOE_ERR_CAPACITY = -4,    /* cap_rows below the worst-case pair count       */
  MOE_ERR_HIP = -5          /* a HIP launch failed (see moe_last_hip_error)   */
} moe_status;

/* MOE_F16 is a router dtype only (moe_route_typed, include/moe_variants.h). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_F16 = 2 } moe_dtype;

/* Expert weight layouts (moe_desc.weight_layout). */
#define MOE_WEIGHTS_STACKED 0 /* gate_up_proj [n, D, 2I], down_proj [n, I, D], act dtype */
#define MOE_WEIGHTS_PACKED 1  /* the operand order moe_pack_expert_weights writes       */

/* Limits of this implementation (MOE_ERR_UNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16
#define MOE_MAX_WIDTH 262144 /* D, I and I_shared */

/*
 * Layer descriptor. The knobs mirror the page "Expert Parallel (EP)",
 * section Configuration: the router runs in fp32 (router_dtype), the router
 * logits can be returned (keep_router_logits), a shared expert can be present
 * (ignore_shared_experts = false), and ep_size logical ranks split the
 * experts evenly (section Requirements: num_experts divisible by ep_size).
 *
 *  T          tokens routed by this rank (>= 0)
 *  D          hidden size (> 0; a multiple of 64; at most MOE_MAX_WIDTH)
 *  E          routed experts, global count (1 .. MOE_MAX_EXPERTS)
 *  top_k      experts per token (1 .. min(E, MOE_MAX_TOPK))
 *  I          routed expert intermediate size (> 0; a multiple of 64; at
 *             most MOE_MAX_WIDTH);
 *             gate_up_proj is [D, 2I], down_proj is [I, D] per expert
 *  ep_size    logical expert-parallel ranks (>= 1, divides E); rank q owns
 *             experts [q*E/ep_size, (q+1)*E/ep_size) (page "Worked Example",
 *             Step 2: expert 11 of 16 on 4 devices is local index 3 of device 2)
 *  ep_rank    this rank (0 .. ep_size-1)
 *  act_dtype  moe_dtype of activations and expert weights
 *  norm_topk  1: routing weights are the chosen experts' softmax probabilities
 *             divided by their sum (they add up to 1, as the 0.6 and 0.4 of
 *             the worked example do); 0: the plain softmax probabilities
 *  I_shared   intermediate size of the one shared expert, 0 for none
 *             (a multiple of 64 when non-zero; at most MOE_MAX_WIDTH)
 *  weight_layout  MOE_WEIGHTS_STACKED (0): expert weights as the stacked
 *             tensors gate_up_proj [n, D, 2I] and down_proj [n, I, D] in the
 *             activation dtype ("tensor-style" experts, page "Expert Parallel
 *             (EP)", Requirements); MOE_WEIGHTS_PACKED (1, bf16 layers only):
 *             the same weights rearranged once by moe_pack_expert_weights.
 *             Every call that reads expert weights (routed and shared) takes
 *             them in this layout; the backward calls and the training forward
 *             take stacked weights only (UNSUPPORTED otherwise).
 *  expert_out_dtype  dtype of the expert outputs y_perm and shared_out that
 *             moe_expert_ffn / moe_expert_down write and moe_unpermute_combine
 *             reads (and of moe_layer_forward's internal copies): MOE_F32 (0,
 *             default), or MOE_F16 for bf16 layers (round to nearest even,
 *             saturating at +-65504; half the bytes of the down GEMM's output
 *             and of the combine's gathers). The backward calls, the training
 *             forward and the MXFP8 FFN take MOE_F32 only (UNSUPPORTED
 *             otherwise).
 */
typedef struct {
  int32_t T, D, E, top_k, I;
  int32_t ep_size, ep_rank;
  int32_t act_dtype;
  int32_t norm_topk;
  int32_t I_shared;
  int32_t weight_layout;
  int32_t expert_out_dtype;
} moe_desc;

/*
 * moe_route - router logits, softmax, top-k and routing weights.
 * Page "Worked Example", Step 1 (logits for all experts, softmax, top-2);
 * page "[Question] How does the gate coordinate across ranks in expert
 * parallelism?" (each rank gates its own local batch with the full
 * [num_experts, embedding_dim] gate weight).
 *
 * The reference logit of token t and expert e is the fp32 rounding of the
 * exact dot product x_t . w_e (plus the bias in fp32). The chosen experts
 * are those of the reference logits exactly (descending, equal logits to
 * the lower expert id), up to the fp64 summation order of the exact path.
 * With fp32 activations, or at most 16 experts, every logit is computed that
 * way (exact products, fp64 sums on the fp64 matrix cores). With bf16
 * activations and more than 16 experts the logits come from the bf16 matrix
 * cores (the gate weight split exactly into three bf16 parts, fp32 sums of
 * at most 128 products), each within a bound the call computes from the row
 * norms; a token whose choice that bound cannot settle gets the reference
 * logits of its candidate experts and is chosen on those.
 *
 *  x          [T, D] act         hidden states
 *  w_router   [E, D] fp32        gate weight
 *  logit_bias [E] fp32 | NULL    added to every token's fp32 logits
 *  logits     [T, E] fp32 | NULL out: the fp32 logits the choice was made on
 *             (after the bias): the reference logits on the fp64 path and
 *             for the recomputed candidates; otherwise within
 *             8.1e-6 ||x_t|| ||w_e|| (plus two fp32 roundings) of them, a
 *             worst case the observed errors stay far below
 *  probs      [T, E] fp32 | NULL out: softmax over all E logits
 *  topk_idx   [T, top_k] int32   out: chosen experts by descending logit;
 *             equal logits go to the lower expert id
 *  topk_w     [T, top_k] fp32    out: routing weights (see norm_topk)
 *  ws         workspace of at least moe_route_workspace_size() bytes (0 on
 *             the fp64 path; ws may then be NULL): partial logits, row norms
 *             and the split gate weight. WORKSPACE if it is smaller.
 */
size_t moe_route_workspace_size(const moe_desc* desc);
moe_status moe_route(const moe_desc* desc, const void* x, const float* w_router,
                     const float* logit_bias, float* logits, float* probs,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * moe_permute - per-expert counts, offsets and split sizes, then an
 * expert-contiguous copy of the (token, expert) pairs whose expert lies in
 * [e_begin, e_end). Page "Expert Parallel (EP)", Communication Pattern,
 * stages 1 (counts and split sizes) and 2 (permute by expert assignment).
 * Rows are ordered by expert, then by ascending token: the order is fixed,
 * so the result is the same on every run.
 *
 *  x          [T, D] act         tokens to permute
 *  topk_idx   [T, top_k] int32   routing (each value in [0, E))
 *  e_begin, e_end  expert range, 0 <= e_begin < e_end <= E; n = e_end-e_begin
 *  cap_rows   rows available in perm_src / x_perm; must be at least
 *             T * min(top_k, n)
 *  counts     [n] int32          out: pairs per in-range expert
 *  offsets    [n + 1] int32      out: exclusive prefix sum of counts
 *  split      [ep_size] int32 | NULL  out: pairs per owning rank
 *  perm_src   [cap_rows] int32   out: source token of row p (rows >= offsets[n]
 *             are left untouched)
 *  pos        [T, top_k] int32   out: row of pair (t, j), -1 if out of range
 *  x_perm     [cap_rows, D] act | NULL  out: x_perm[p] = x[perm_src[p]]
 *  ws         workspace of at least moe_permute_workspace_size() bytes
 */
moe_status moe_permute(const moe_desc* desc, const void* x, const int32_t* topk_idx,
                       int32_t e_begin, int32_t e_end, int64_t cap_rows,
                       int32_t* counts, int32_t* offsets, int32_t* split,
                       int32_t* perm_src, int32_t* pos, void* x_perm,
                       void* ws, size_t ws_bytes, void* stream);
size_t moe_permute_workspace_size(const moe_desc* desc, int32_t e_begin, int32_t e_end);

/*
 * moe_permute_noalloc - moe_permute without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops that must not call hipMalloc, harnesses that forbid it). Same
 * arguments (minus ws / ws_bytes), results and errors as moe_permute; the
 * result is bit-identical to moe_permute's.
 *
 * Its scratch (the per-block expert counts and first rows) lives in a
 * file-scope device array of the library, 96 KB on each GPU the call runs
 * on, held until the process ends; the permute's scratch never exceeds it
 * (token blocks grow so that blocks x experts stays within 12288), and a
 * call that would need more returns MOE_ERR_WORKSPACE. The array's device
 * address is looked up once per device (hipGetSymbolAddress) on the first
 * call made with that device current. The call allocates and frees nothing.
 * Every call on one GPU uses the same array: calls that overlap on one GPU
 * (different streams, or host threads) race and must be ordered by the
 * caller; consecutive calls on one stream are safe (each writes every
 * scratch entry it reads before reading it).
 */
moe_status moe_permute_noalloc(const moe_desc* desc, const void* x, const int32_t* topk_idx,
                               int32_t e_begin, int32_t e_end, int64_t cap_rows,
                               int32_t* counts, int32_t* offsets, int32_t* split,
                               int32_t* perm_src, int32_t* pos, void* x_perm, void* stream);

/*
 * moe_expert_ffn - every local expert's two-layer SiLU-gated feed-forward on
 * its segment of rows: H = SiLU(X W_gate) * (X W_up), Y = H W_down, where
 * W_gate and W_up are columns [0, I) and [I, 2I) of gate_up_proj.
 * Page "Expert Parallel (EP)", Communication Pattern stage 3 and Requirements
 * (tensor-style gate_up_proj / down_proj); page "Worked Example", Step 3.
 * bf16 layers: fp32 accumulation on the matrix cores; H is kept in fp16 in
 * the workspace and the down projection runs in fp16 with down_proj
 * converted from bf16 (round to nearest even) on the fly; Y is fp32.
 * fp16 holds magnitudes up to 65504: an H value beyond that saturates to
 * +-65504 (a finite H never becomes infinite; NaN stays NaN), so Y and the
 * layer output stay finite but are clipped for such rows. Unit-scale
 * hidden states with 0.02-scale weights keep |H| orders of magnitude below
 * that bound.
 * fp32 layers: fp32 throughout.
 *
 *  n_experts  local experts (1 .. MOE_MAX_EXPERTS)
 *  inter      intermediate size I of these experts (desc->I for routed
 *             experts, desc->I_shared for the shared one)
 *  cap_rows   rows of x_perm / y_perm
 *  x_perm     [cap_rows, D] act
 *  offsets    [n_experts + 1] int32 DEVICE | NULL: expert j owns rows
 *             [offsets[j], offsets[j+1]); NULL means one expert owning all
 *             cap_rows rows (a dense FFN, used for the shared expert), and
 *             then n_experts must be 1 (INVALID_ARG otherwise)
 *  w_gate_up  [n_experts, D, 2*inter] act
 *  w_down     [n_experts, inter, D] act
 *  y_perm     [cap_rows, D] fp32, or fp16 (expert_out_dtype)  out (rows past
 *             offsets[n] untouched)
 *  ws         workspace of at least moe_ffn_workspace_size() bytes: H, and
 *             for bf16 layers the down GEMM's part buffer (see moe_expert_down)
 */
moe_status moe_expert_ffn(const moe_desc* desc, int32_t n_experts, int32_t inter,
                          int64_t cap_rows, const void* x_perm, const int32_t* offsets,
                          const void* w_gate_up, const void* w_down, void* y_perm,
                          void* ws, size_t ws_bytes, void* stream);
size_t moe_ffn_workspace_size(const moe_desc* desc, int32_t inter, int64_t cap_rows);

/*
 * The two halves of moe_expert_ffn, for callers that keep H themselves.
 * moe_expert_gate_up: the grouped gate_up GEMM with the SiLU-gate epilogue,
 *   h[r, c] = SiLU(x_perm[r] . W_gate[:, c]) * (x_perm[r] . W_up[:, c]);
 *   page "Worked Example", Step 3 (first layer of the expert FFN); the gated
 *   activation is the one the tensor-style gate_up_proj of page "Expert
 *   Parallel (EP)", Requirements, implies.
 * moe_expert_down: the grouped down GEMM, y_perm = h . W_down (second layer).
 *
 *  h       [cap_rows, inter]: fp16 (raw 16-bit words) for bf16 layers,
 *          fp32 for fp32 layers; written by gate_up, read by down
 *  ws      NULL (ws_bytes ignored): every tile runs whole. Or a buffer of at
 *          least moe_gate_up_workspace_size() / moe_down_workspace_size()
 *          bytes (bf16 layers; gate_up with MOE_WEIGHTS_PACKED only): when
 *          the 256 x 256 tiles need a last, partial round over the CUs, that
 *          round's tiles are cut along K into parts whose fp32 sums land in
 *          ws and a second launch adds them in part order (a fixed order:
 *          the same bits every call; against whole tiles only the order of
 *          the fp32 sums differs) and, for gate_up, applies the SiLU gate.
 *          moe_expert_ffn and moe_layer_forward do the same in their own
 *          workspace. WORKSPACE if ws_bytes is smaller.
 *  other arguments as for moe_expert_ffn (y_perm in expert_out_dtype)
 */
moe_status moe_expert_gate_up(const moe_desc* desc, int32_t n_experts, int32_t inter,
                              int64_t cap_rows, const void* x_perm, const int32_t* offsets,
                              const void* w_gate_up, void* h, void* ws, size_t ws_bytes,
                              void* stream);
moe_status moe_expert_down(const moe_desc* desc, int32_t n_experts, int32_t inter,
                           int64_t cap_rows, const void* h, const int32_t* offsets,
                           const void* w_down, void* y_perm, void* ws, size_t ws_bytes,
                           void* stream);
/* Part buffer bytes moe_expert_gate_up (inter H columns) and moe_expert_down
 * may use for cap_rows rows (0 for fp32 layers, and 0 from
 * moe_gate_up_workspace_size for an invalid desc or inter < 1). Host
 * arithmetic. */
size_t moe_gate_up_workspace_size(const moe_desc* desc, int32_t inter, int64_t cap_rows);
size_t moe_down_workspace_size(const moe_desc* desc, int64_t cap_rows);

/*
 * moe_pack_expert_weights - rearrange stacked bf16 expert weights once (at
 * weight-load time) into the order in which the grouped GEMMs feed the
 * matrix cores, for calls with weight_layout = MOE_WEIGHTS_PACKED. Same
 * weights as the tensor-style gate_up_proj / down_proj of page "Expert
 * Parallel (EP)", Requirements; only their order in memory (and down_proj's
 * 16-bit format) differs.
 *
 * For a stacked [n, K, N] weight, the packed buffer holds, for expert e,
 * 32-column block cb, 16-deep slice ks of K, lane l (0..63) and j (0..7),
 *   packed[e][cb][ks][l][j] = w[e][16 ks + 8 (l / 32) + j][32 cb + l % 32]:
 * each 1 KB (cb, ks) fragment is one matrix-core operand, K contiguous per
 * lane, so a workgroup copies it with one instruction and reads it with one
 * 16-byte LDS read per lane.
 *
 *  n_experts, inter   as for moe_expert_ffn (desc->D is the hidden size)
 *  w_gate_up       [n, D, 2 inter] bf16 | NULL (stacked)
 *  w_down          [n, inter, D] bf16 | NULL (stacked)
 *  packed_gate_up  out: n * D * 2 inter bf16 values (NULL iff w_gate_up is)
 *  packed_down     out: n * inter * D fp16 values, each bf16 value rounded to
 *                  nearest even (exact for |w| in [2^-14, 65504]; the stacked
 *                  down GEMM makes the same conversion as it reads, so both
 *                  layouts give identical results) (NULL iff w_down is)
 * The packed buffers must not overlap the stacked ones. bf16 layers only
 * (UNSUPPORTED otherwise); n_experts = 1 packs a shared expert's weights.
 */
moe_status moe_pack_expert_weights(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                   const void* w_gate_up, const void* w_down,
                                   void* packed_gate_up, void* packed_down, void* stream);

/*
 * moe_ffn_tile_shape - the workgroup tile the grouped GEMMs of moe_expert_ffn
 * (and its two halves) take for these sizes: host arithmetic only, no HIP
 * call beyond reading the device's compute-unit count once (256 when no GPU
 * is visible). The choice depends on cap_rows, never on the offsets' values.
 *
 *  n_experts, inter, cap_rows   as for moe_expert_ffn
 *  has_offsets  1: the experts' segments come from device offsets; 0: one
 *               dense expert (offsets == NULL; n_experts must be 1)
 *  gemm         0: the gate_up GEMM, 1: the down GEMM
 *  tile_rows    out: rows per tile (256 or 320 for bf16 layers; 64 for fp32)
 *  tile_cols    out: product columns per tile (gate and up columns together
 *               for the gate_up GEMM)
 * Errors: as moe_expert_ffn's argument checks; INVALID_ARG for another
 * gemm value or a NULL output.
 */
moe_status moe_ffn_tile_shape(const moe_desc* desc, int32_t n_experts, int32_t inter,
                              int64_t cap_rows, int32_t has_offsets, int32_t gemm,
                              int32_t* tile_rows, int32_t* tile_cols);

/*
 * moe_unpermute_combine - out[t] = residual[t] + shared[t]
 *                                  + sum_j topk_w[t,j] * y_perm[pos[t,j]],
 * skipping slots with pos < 0. Page "Expert Parallel (EP)", Communication
 * Pattern stage 4 (unpermute and apply routing weights); page "Worked
 * Example", Step 4 (weighted sum of expert outputs) and Step 5 (residual).
 * Accumulates in fp32 and rounds once to the output dtype.
 *
 *  y_perm     [rows, D] expert_out_dtype  expert outputs (rows >= max pos + 1)
 *  pos        [T, top_k] int32
 *  topk_w     [T, top_k] fp32
 *  residual   [res_rows, D] act | NULL   added to out rows [res_begin, res_begin+res_rows)
 *  shared_out [res_rows, D] expert_out_dtype | NULL  added to the same rows
 *  res_begin, res_rows   0 <= res_begin, res_begin + res_rows <= T
 *  out        [T, D] act         out
 */
moe_status moe_unpermute_combine(const moe_desc* desc, const void* y_perm,
                                 const int32_t* pos, const float* topk_w,
                                 const void* residual, const void* shared_out,
                                 int32_t res_begin, int32_t res_rows,
                                 void* out, void* stream);

/*
 * moe_layer_forward - the whole layer on this GPU: route the T tokens, count
 * and split over ep_size logical ranks, permute, run all E experts, add the
 * shared expert (when I_shared > 0) and combine into the residual:
 *   out = x + shared(x) + sum_j w_j * expert_{idx_j}(x).
 * Page "Expert Parallel (EP)", Communication Pattern (the four stages:
 * preprocess with counts and split sizes, permute by expert, expert compute,
 * unpermute with routing weights; the all-to-alls between them are left out,
 * every expert being local); page "Worked Example: Tracing a Token Through
 * Expert Parallelism", Steps 1-5 (router and top-k, dispatch by local expert
 * index, expert FFN, weighted sum, residual). The shared-expert term follows
 * torchtitan issue 5554: the shared expert's output is added unweighted to
 * the routed sum before the combination.
 * Every expert is computed here; split reports the pair counts each logical
 * rank would receive.
 *
 *  x [T, D] act; w_router [E, D] fp32; logit_bias [E] fp32 | NULL
 *  w_gate_up [E, D, 2I] act; w_down [E, I, D] act
 *  shared_gate_up [D, 2*I_shared] act | NULL; shared_down [I_shared, D] act | NULL
 *  out [T, D] act                 out
 *  logits [T, E] fp32 | NULL      out
 *  topk_idx [T, top_k] int32, topk_w [T, top_k] fp32   out
 *  counts [E] int32, offsets [E + 1] int32             out
 *  split [ep_size] int32 | NULL                        out
 *  perm_src [T * top_k] int32 | NULL, pos [T, top_k] int32 | NULL  out
 *  ws   workspace of at least moe_workspace_size() bytes
 */
moe_status moe_layer_forward(const moe_desc* desc, const void* x, const float* w_router,
                             const float* logit_bias, const void* w_gate_up,
                             const void* w_down, const void* shared_gate_up,
                             const void* shared_down, void* out, float* logits,
                             int32_t* topk_idx, float* topk_w, int32_t* counts,
                             int32_t* offsets, int32_t* split, int32_t* perm_src,
                             int32_t* pos, void* ws, size_t ws_bytes, void* stream);
size_t moe_workspace_size(const moe_desc* desc);

/* Human-readable name of a status code (static storage). */
const char* moe_status_str(int32_t status);

/* hipError_t of the last failed launch on the calling thread (0 = none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
