// C ABI of libmoe: argument checks, workspace sizing and launch sequencing.
//
// Every check below is host arithmetic on the descriptor and on pointer
// nullness and runs before any HIP call, so a rejected call needs no GPU.
// The library allocates nothing, keeps no pointer and never synchronises.
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "moe_internal.h"
#include "moe_backward.h"
#include "moe_mxfp8.h"
#include "moe_variants.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local int32_t g_last_hip_error = 0;

inline size_t align_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

inline size_t act_bytes(const moe_desc& d) { return d.act_dtype == MOE_BF16 ? 2 : 4; }

moe_status check_desc(const moe_desc* d) {
  if (d == nullptr) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->D <= 0 || d->E < 1 || d->top_k < 1 || d->top_k > d->E || d->I <= 0 ||
      d->ep_size < 1 || d->ep_rank < 0 || d->ep_rank >= d->ep_size || d->I_shared < 0 ||
      (d->norm_topk != 0 && d->norm_topk != 1))
    return MOE_ERR_INVALID_ARG;
  // Page "Expert Parallel (EP)", Requirements: num_experts divisible by ep_size.
  if (d->E % d->ep_size != 0) return MOE_ERR_INVALID_ARG;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->E > MOE_MAX_EXPERTS || d->top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (d->D % 64 != 0 || d->I % 64 != 0 || d->I_shared % 64 != 0) return MOE_ERR_UNSUPPORTED;
  // The grouped GEMMs address a tile's rows of an output with 32-bit offsets.
  if (d->D > MOE_MAX_WIDTH || d->I > MOE_MAX_WIDTH || d->I_shared > MOE_MAX_WIDTH)
    return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(d->T) * d->top_k > INT_MAX) return MOE_ERR_UNSUPPORTED;
  if (d->weight_layout != MOE_WEIGHTS_STACKED && d->weight_layout != MOE_WEIGHTS_PACKED)
    return MOE_ERR_INVALID_ARG;
  if (d->weight_layout == MOE_WEIGHTS_PACKED && d->act_dtype != MOE_BF16)
    return MOE_ERR_UNSUPPORTED;
  if (d->expert_out_dtype != MOE_F32 && d->expert_out_dtype != MOE_F16) return MOE_ERR_INVALID_ARG;
  if (d->expert_out_dtype == MOE_F16 && d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline bool packed(const moe_desc& d) { return d.weight_layout == MOE_WEIGHTS_PACKED; }
inline bool y_half(const moe_desc& d) { return d.expert_out_dtype == MOE_F16; }

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int32_t>(e);
  return MOE_ERR_HIP;
}

size_t permute_ws(const moe_desc& d, int n) {
  const int pb = moe::perm_token_block(d.T, n);
  const size_t nb = static_cast<size_t>((d.T + pb - 1) / pb);
  return 2 * align_up(nb * n * sizeof(int32_t));
}

// FFN workspace: H between the two GEMMs (fp16 for bf16 layers, fp32 for
// fp32 layers), then for bf16 layers the split-K part buffer the two GEMMs
// use in turn.
size_t ffn_h_bytes(const moe_desc& d, int inter, int64_t cap_rows) {
  return align_up(static_cast<size_t>(cap_rows) * inter * act_bytes(d));
}
size_t tail_bytes(const moe_desc& d, int64_t cap_rows) {  // the down GEMM's
  return d.act_dtype == MOE_BF16 ? align_up(moe::down_tail_bytes(cap_rows, d.E, d.D)) : 0;
}
size_t gate_up_tail_bytes(const moe_desc& d, int inter, int64_t cap_rows) {
  return d.act_dtype == MOE_BF16 ? align_up(moe::gate_up_tail_bytes(cap_rows, d.E, inter)) : 0;
}
size_t ffn_tail_bytes(const moe_desc& d, int inter, int64_t cap_rows) {
  return std::max(tail_bytes(d, cap_rows), gate_up_tail_bytes(d, inter, cap_rows));
}
size_t ffn_ws(const moe_desc& d, int inter, int64_t cap_rows) {
  return ffn_h_bytes(d, inter, cap_rows) + ffn_tail_bytes(d, inter, cap_rows);
}

// Expert outputs (y_perm, shared expert output): fp16 or fp32.
inline size_t out_bytes(const moe_desc& d) { return d.expert_out_dtype == MOE_F16 ? 2 : 4; }

// Layer workspace: permute scratch, perm_src, pos, x_perm, H, y_perm, and for a
// shared expert its H and output.
struct LayerWs {
  size_t perm, perm_src, pos, x_perm, h, y_perm, h_sh, s_out, tail, tail_bytes, total;
};

LayerWs layer_ws(const moe_desc& d) {
  LayerWs w{};
  const size_t M = static_cast<size_t>(d.T) * d.top_k;
  const size_t s = act_bytes(d);
  size_t o = 0;
  w.perm = o;      o += permute_ws(d, d.E);
  w.perm_src = o;  o += align_up(M * sizeof(int32_t));
  w.pos = o;       o += align_up(M * sizeof(int32_t));
  w.x_perm = o;    o += align_up(M * d.D * s);
  // H is written after the router is done with its scratch, which lives here.
  w.h = o;         o += align_up(std::max(M * d.I * s, moe::route_ws_bytes(d)));
  w.y_perm = o;    o += align_up(M * d.D * out_bytes(d));
  w.h_sh = o;      o += align_up(static_cast<size_t>(d.T) * d.I_shared * s);
  w.s_out = o;     o += d.I_shared > 0 ? align_up(static_cast<size_t>(d.T) * d.D * out_bytes(d)) : 0;
  w.tail = o;
  w.tail_bytes = std::max(ffn_tail_bytes(d, d.I, static_cast<int64_t>(M)),
                          d.I_shared > 0 ? ffn_tail_bytes(d, d.I_shared, d.T) : 0);
  o += w.tail_bytes;
  w.total = o;
  return w;
}

// tail: the split-K part buffer (tail_n bytes), or null.
hipError_t run_gate_up(const moe_desc& d, int n_experts, int64_t cap_rows, int inter,
                       const void* x_perm, const int32_t* offsets, const void* w_gate_up, void* h,
                       hipStream_t s, void* tail = nullptr, size_t tail_n = 0) {
  if (d.act_dtype == MOE_BF16)
    return moe::launch_gate_up_bf16(n_experts, cap_rows, d.D, inter, x_perm, offsets, w_gate_up, h,
                                    s, nullptr, packed(d), tail, tail_n);
  return moe::launch_gate_up_f32(n_experts, cap_rows, d.D, inter, x_perm, offsets, w_gate_up, h, s);
}

// tail: the down GEMM's split-K part buffer (tail_n bytes), or null.
hipError_t run_down(const moe_desc& d, int n_experts, int64_t cap_rows, int inter, const void* h,
                    const int32_t* offsets, const void* w_down, void* y, hipStream_t s,
                    void* tail = nullptr, size_t tail_n = 0) {
  if (d.act_dtype == MOE_BF16)
    return moe::launch_down_bf16(n_experts, cap_rows, d.D, inter, h, offsets, w_down, y, s, nullptr,
                                 packed(d), y_half(d), tail, tail_n);
  return moe::launch_down_f32(n_experts, cap_rows, d.D, inter, h, offsets, w_down, y, s);
}

hipError_t run_ffn(const moe_desc& d, int n_experts, int64_t cap_rows, int inter,
                   const void* x_perm, const int32_t* offsets, const void* w_gate_up,
                   const void* w_down, void* h, void* y, hipStream_t s, void* tail,
                   size_t tail_n) {
  hipError_t e =
      run_gate_up(d, n_experts, cap_rows, inter, x_perm, offsets, w_gate_up, h, s, tail, tail_n);
  if (e != hipSuccess) return e;
  return run_down(d, n_experts, cap_rows, inter, h, offsets, w_down, y, s, tail, tail_n);
}

moe_status check_ffn_args(const moe_desc* desc, int32_t n_experts, int32_t inter,
                          int64_t cap_rows) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (n_experts < 1 || inter <= 0 || cap_rows < 0) return MOE_ERR_INVALID_ARG;
  if (n_experts > MOE_MAX_EXPERTS || inter % 64 != 0 || cap_rows > INT_MAX)
    return MOE_ERR_UNSUPPORTED;
  // The grouped GEMMs address one expert's weight matrix with 32-bit byte
  // offsets kept below 2^30.
  if (static_cast<int64_t>(desc->D) * inter * 4 >= (int64_t(1) << 30))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

MOE_API const char* moe_status_str(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_CAPACITY: return "row capacity too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

MOE_API int32_t moe_last_hip_error(void) { return g_last_hip_error; }

MOE_API size_t moe_route_workspace_size(const moe_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return moe::route_ws_bytes(*desc);
}

MOE_API moe_status moe_route(const moe_desc* desc, const void* x, const float* w_router,
                             const float* logit_bias, float* logits, float* probs,
                             int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                             void* stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (x == nullptr || w_router == nullptr || topk_idx == nullptr || topk_w == nullptr)
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe::route_ws_bytes(*desc);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route(*desc, x, w_router, logit_bias, logits, probs, topk_idx,
                                      topk_w, ws, static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_route_typed(const moe_desc* desc, int32_t router_dtype, const void* x,
                                   const void* w_router, const float* logit_bias, void* logits,
                                   float* probs, int32_t* topk_idx, float* topk_w, void* stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (router_dtype != MOE_F32 && router_dtype != MOE_BF16 && router_dtype != MOE_F16)
    return MOE_ERR_INVALID_ARG;
  if (desc->T == 0) return MOE_OK;
  if (x == nullptr || w_router == nullptr || topk_idx == nullptr || topk_w == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_route_typed(*desc, router_dtype, x, w_router, logit_bias, logits,
                                            probs, topk_idx, topk_w,
                                            static_cast<hipStream_t>(stream)));
}

MOE_API size_t moe_permute_workspace_size(const moe_desc* desc, int32_t e_begin, int32_t e_end) {
  if (check_desc(desc) != MOE_OK || e_begin < 0 || e_end <= e_begin || e_end > desc->E) return 0;
  return permute_ws(*desc, e_end - e_begin);
}

namespace {
// Checks of moe_permute's arguments (all but the workspace).
moe_status check_permute_args(const moe_desc* desc, const void* x, const int32_t* topk_idx,
                              int32_t e_begin, int32_t e_end, int64_t cap_rows,
                              const int32_t* counts, const int32_t* offsets,
                              const int32_t* perm_src, const int32_t* pos, const void* x_perm) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (e_begin < 0 || e_end <= e_begin || e_end > desc->E) return MOE_ERR_INVALID_ARG;
  if (counts == nullptr || offsets == nullptr) return MOE_ERR_INVALID_ARG;
  if (desc->T > 0 && (topk_idx == nullptr || perm_src == nullptr || pos == nullptr ||
                      (x_perm != nullptr && x == nullptr)))
    return MOE_ERR_INVALID_ARG;
  const int n = e_end - e_begin;
  const int64_t need = static_cast<int64_t>(desc->T) * (desc->top_k < n ? desc->top_k : n);
  if (cap_rows < need || cap_rows > INT_MAX) return MOE_ERR_CAPACITY;
  return MOE_OK;
}

// The permute's scratch: per-block counts at ws, per-block first rows after them.
hipError_t run_permute(const moe_desc& d, const void* x, const int32_t* topk_idx, int e_begin,
                       int e_end, int32_t* counts, int32_t* offsets, int32_t* split,
                       int32_t* perm_src, int32_t* pos, void* x_perm, void* ws, hipStream_t s) {
  const int n = e_end - e_begin;
  const int pb = moe::perm_token_block(d.T, n);
  const size_t nb = static_cast<size_t>((d.T + pb - 1) / pb);
  int32_t* block_counts = static_cast<int32_t*>(ws);
  int32_t* block_base = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                                   align_up(nb * n * sizeof(int32_t)));
  return moe::launch_permute(d, x, topk_idx, e_begin, e_end, counts, offsets, split, perm_src, pos,
                             x_perm, block_counts, block_base, s);
}
}  // namespace

MOE_API moe_status moe_permute(const moe_desc* desc, const void* x, const int32_t* topk_idx,
                               int32_t e_begin, int32_t e_end, int64_t cap_rows,
                               int32_t* counts, int32_t* offsets, int32_t* split,
                               int32_t* perm_src, int32_t* pos, void* x_perm, void* ws,
                               size_t ws_bytes, void* stream) {
  moe_status st = check_permute_args(desc, x, topk_idx, e_begin, e_end, cap_rows, counts,
                                     offsets, perm_src, pos, x_perm);
  if (st != MOE_OK) return st;
  if (ws == nullptr) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < permute_ws(*desc, e_end - e_begin)) return MOE_ERR_WORKSPACE;
  return hip_status(run_permute(*desc, x, topk_idx, e_begin, e_end, counts, offsets, split,
                                perm_src, pos, x_perm, ws, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// moe_permute_noalloc: moe_permute with its scratch in a file-scope device
// array instead of a caller workspace (for callers that cannot allocate).
// ---------------------------------------------------------------------------
// Per-block counts, then per-block first rows: the whole scratch the permute
// needs for any T and expert range (perm_token_block keeps blocks x experts
// within kPermMaxBlockCounts). 96 KB per device, held until the process ends.
static __device__ __align__(256) int32_t scratch[2 * moe::kPermMaxBlockCounts];

namespace {

constexpr size_t kPermScratchBytes = sizeof(scratch);

// The array's device address, looked up once per device (each device holds
// its own copy). In host code `scratch` only names a host-side stand-in; the
// kernels get this address instead.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

MOE_API moe_status moe_permute_noalloc(const moe_desc* desc, const void* x,
                                       const int32_t* topk_idx, int32_t e_begin, int32_t e_end,
                                       int64_t cap_rows, int32_t* counts, int32_t* offsets,
                                       int32_t* split, int32_t* perm_src, int32_t* pos,
                                       void* x_perm, void* stream) {
  moe_status st = check_permute_args(desc, x, topk_idx, e_begin, e_end, cap_rows, counts,
                                     offsets, perm_src, pos, x_perm);
  if (st != MOE_OK) return st;
  if (permute_ws(*desc, e_end - e_begin) > kPermScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_status(e);
  // Every entry of the scratch the kernels read is written earlier in the
  // same call (counts by the count kernel, first rows by the scan), so no
  // clearing is needed; calls that overlap on one device share the array and
  // race.
  return hip_status(run_permute(*desc, x, topk_idx, e_begin, e_end, counts, offsets, split,
                                perm_src, pos, x_perm, ws, static_cast<hipStream_t>(stream)));
}

MOE_API size_t moe_ffn_workspace_size(const moe_desc* desc, int32_t inter, int64_t cap_rows) {
  if (check_desc(desc) != MOE_OK || inter <= 0 || cap_rows < 0) return 0;
  return ffn_ws(*desc, inter, cap_rows);
}

MOE_API moe_status moe_expert_ffn(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                  int64_t cap_rows, const void* x_perm, const int32_t* offsets,
                                  const void* w_gate_up, const void* w_down, void* y_perm,
                                  void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_args(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (offsets == nullptr && n_experts != 1) return MOE_ERR_INVALID_ARG;
  if (cap_rows == 0) return MOE_OK;
  if (x_perm == nullptr || w_gate_up == nullptr || w_down == nullptr || y_perm == nullptr ||
      ws == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_ws(*desc, inter, cap_rows)) return MOE_ERR_WORKSPACE;
  return hip_status(run_ffn(*desc, n_experts, cap_rows, inter, x_perm, offsets, w_gate_up, w_down,
                            ws, y_perm, static_cast<hipStream_t>(stream),
                            static_cast<char*>(ws) + ffn_h_bytes(*desc, inter, cap_rows),
                            ffn_tail_bytes(*desc, inter, cap_rows)));
}

MOE_API moe_status moe_expert_ffn_train(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                        int64_t cap_rows, const void* x_perm,
                                        const int32_t* offsets, const void* w_gate_up,
                                        const void* w_down, void* y_perm, float* gu_saved,
                                        void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_args(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (desc->act_dtype != MOE_BF16 || packed(*desc) || y_half(*desc)) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr && n_experts != 1) return MOE_ERR_INVALID_ARG;
  if (cap_rows == 0) return MOE_OK;
  if (x_perm == nullptr || w_gate_up == nullptr || w_down == nullptr || y_perm == nullptr ||
      gu_saved == nullptr || ws == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_ws(*desc, inter, cap_rows)) return MOE_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = moe::launch_gate_up_save_bf16(n_experts, cap_rows, desc->D, inter, x_perm,
                                               offsets, w_gate_up, ws, gu_saved, s);
  if (e == hipSuccess)
    e = moe::launch_down_bf16(n_experts, cap_rows, desc->D, inter, ws, offsets, w_down, y_perm, s,
                              nullptr, false, false,
                              static_cast<char*>(ws) + ffn_h_bytes(*desc, inter, cap_rows),
                              tail_bytes(*desc, cap_rows));
  return hip_status(e);
}

MOE_API moe_status moe_expert_ffn_ptrs(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                       int64_t cap_rows, const void* x_perm,
                                       const int32_t* offsets, const void* const* w_gate_up_ptrs,
                                       const void* const* w_down_ptrs, void* y_perm, void* ws,
                                       size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_args(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (desc->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr && n_experts != 1) return MOE_ERR_INVALID_ARG;
  if (cap_rows == 0) return MOE_OK;
  if (x_perm == nullptr || w_gate_up_ptrs == nullptr || w_down_ptrs == nullptr ||
      y_perm == nullptr || ws == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_ws(*desc, inter, cap_rows)) return MOE_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* tail = static_cast<char*>(ws) + ffn_h_bytes(*desc, inter, cap_rows);
  const size_t tail_n = ffn_tail_bytes(*desc, inter, cap_rows);
  hipError_t e = moe::launch_gate_up_bf16(n_experts, cap_rows, desc->D, inter, x_perm, offsets,
                                          nullptr, ws, s, w_gate_up_ptrs, packed(*desc), tail,
                                          tail_n);
  if (e == hipSuccess)
    e = moe::launch_down_bf16(n_experts, cap_rows, desc->D, inter, ws, offsets, nullptr, y_perm, s,
                              w_down_ptrs, packed(*desc), y_half(*desc), tail, tail_n);
  return hip_status(e);
}

MOE_API moe_status moe_pack_expert_weights(const moe_desc* desc, int32_t n_experts,
                                           int32_t inter, const void* w_gate_up,
                                           const void* w_down, void* packed_gate_up,
                                           void* packed_down, void* stream) {
  moe_status st = check_ffn_args(desc, n_experts, inter, 0);
  if (st != MOE_OK) return st;
  if (desc->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if ((w_gate_up == nullptr) != (packed_gate_up == nullptr) ||
      (w_down == nullptr) != (packed_down == nullptr) ||
      (w_gate_up != nullptr && w_gate_up == packed_gate_up) ||
      (w_down != nullptr && w_down == packed_down))
    return MOE_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (w_gate_up != nullptr)
    e = moe::launch_pack_weights(n_experts, desc->D, 2 * inter, false, w_gate_up, packed_gate_up,
                                 s);
  if (e == hipSuccess && w_down != nullptr)
    e = moe::launch_pack_weights(n_experts, inter, desc->D, true, w_down, packed_down, s);
  return hip_status(e);
}

MOE_API moe_status moe_ffn_tile_shape(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                      int64_t cap_rows, int32_t has_offsets, int32_t gemm,
                                      int32_t* tile_rows, int32_t* tile_cols) {
  moe_status st = check_ffn_args(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if ((gemm != 0 && gemm != 1) || tile_rows == nullptr || tile_cols == nullptr ||
      (has_offsets != 0 && has_offsets != 1) || (!has_offsets && n_experts != 1))
    return MOE_ERR_INVALID_ARG;
  if (desc->act_dtype != MOE_BF16) {  // the fp32 SIMT kernels' 64 x 64 tiles
    *tile_rows = 64;
    *tile_cols = gemm == 0 ? 128 : 64;
    return MOE_OK;
  }
  int r = 0, c = 0;
  moe::ffn_tile_shape_bf16(n_experts, cap_rows, desc->D, inter, has_offsets != 0, gemm, &r, &c);
  *tile_rows = r;
  *tile_cols = c;
  return MOE_OK;
}

MOE_API size_t moe_gate_up_workspace_size(const moe_desc* desc, int32_t inter,
                                          int64_t cap_rows) {
  if (check_desc(desc) != MOE_OK || cap_rows < 0 || inter < 1) return 0;
  return gate_up_tail_bytes(*desc, inter, cap_rows);
}

MOE_API moe_status moe_expert_gate_up(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                      int64_t cap_rows, const void* x_perm,
                                      const int32_t* offsets, const void* w_gate_up, void* h,
                                      void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_args(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (offsets == nullptr && n_experts != 1) return MOE_ERR_INVALID_ARG;
  if (cap_rows == 0) return MOE_OK;
  if (x_perm == nullptr || w_gate_up == nullptr || h == nullptr) return MOE_ERR_INVALID_ARG;
  const size_t tb = gate_up_tail_bytes(*desc, inter, cap_rows);
  if (ws != nullptr && ws_bytes < tb) return MOE_ERR_WORKSPACE;
  return hip_status(run_gate_up(*desc, n_experts, cap_rows, inter, x_perm, offsets, w_gate_up, h,
                                static_cast<hipStream_t>(stream), ws, ws != nullptr ? tb : 0));
}

MOE_API size_t moe_down_workspace_size(const moe_desc* desc, int64_t cap_rows) {
  if (check_desc(desc) != MOE_OK || cap_rows < 0) return 0;
  return tail_bytes(*desc, cap_rows);
}

MOE_API moe_status moe_expert_down(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                   int64_t cap_rows, const void* h, const int32_t* offsets,
                                   const void* w_down, void* y_perm, void* ws, size_t ws_bytes,
                                   void* stream) {
  moe_status st = check_ffn_args(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (offsets == nullptr && n_experts != 1) return MOE_ERR_INVALID_ARG;
  if (cap_rows == 0) return MOE_OK;
  if (h == nullptr || w_down == nullptr || y_perm == nullptr) return MOE_ERR_INVALID_ARG;
  const size_t tb = tail_bytes(*desc, cap_rows);
  if (ws != nullptr && ws_bytes < tb) return MOE_ERR_WORKSPACE;
  return hip_status(run_down(*desc, n_experts, cap_rows, inter, h, offsets, w_down, y_perm,
                             static_cast<hipStream_t>(stream), ws, ws != nullptr ? tb : 0));
}

MOE_API moe_status moe_unpermute_combine(const moe_desc* desc, const void* y_perm,
                                         const int32_t* pos, const float* topk_w,
                                         const void* residual, const void* shared_out,
                                         int32_t res_begin, int32_t res_rows, void* out,
                                         void* stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (res_begin < 0 || res_rows < 0 || static_cast<int64_t>(res_begin) + res_rows > desc->T)
    return MOE_ERR_INVALID_ARG;
  if (desc->T == 0) return MOE_OK;
  if (pos == nullptr || topk_w == nullptr || out == nullptr || y_perm == nullptr)
    return MOE_ERR_INVALID_ARG;
  if ((residual != nullptr || shared_out != nullptr) && res_rows == 0) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(*desc, y_perm, pos, topk_w, residual, shared_out,
                                        res_begin, res_rows, out,
                                        static_cast<hipStream_t>(stream)));
}

MOE_API size_t moe_workspace_size(const moe_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return layer_ws(*desc).total;
}

MOE_API moe_status moe_layer_forward(const moe_desc* desc, const void* x, const float* w_router,
                                     const float* logit_bias, const void* w_gate_up,
                                     const void* w_down, const void* shared_gate_up,
                                     const void* shared_down, void* out, float* logits,
                                     int32_t* topk_idx, float* topk_w, int32_t* counts,
                                     int32_t* offsets, int32_t* split, int32_t* perm_src,
                                     int32_t* pos, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  const moe_desc& d = *desc;
  if (counts == nullptr || offsets == nullptr || ws == nullptr) return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (x == nullptr || w_router == nullptr || w_gate_up == nullptr ||
                  w_down == nullptr || out == nullptr || topk_idx == nullptr || topk_w == nullptr))
    return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && d.I_shared > 0 && (shared_gate_up == nullptr || shared_down == nullptr))
    return MOE_ERR_INVALID_ARG;
  const LayerWs lw = layer_ws(d);
  if (ws_bytes < lw.total) return MOE_ERR_WORKSPACE;
  if (static_cast<int64_t>(d.D) * d.I * 4 >= (int64_t(1) << 30) ||
      static_cast<int64_t>(d.D) * d.I_shared * 4 >= (int64_t(1) << 30))
    return MOE_ERR_UNSUPPORTED;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const int64_t M = static_cast<int64_t>(d.T) * d.top_k;
  int32_t* ps = perm_src ? perm_src : reinterpret_cast<int32_t*>(base + lw.perm_src);
  int32_t* pp = pos ? pos : reinterpret_cast<int32_t*>(base + lw.pos);
  void* x_perm = base + lw.x_perm;
  void* h = base + lw.h;
  void* y_perm = base + lw.y_perm;

  hipError_t e = hipSuccess;
  if (d.T > 0) {
    e = moe::launch_route(d, x, w_router, logit_bias, logits, nullptr, topk_idx, topk_w, h, s);
    if (e != hipSuccess) return hip_status(e);
  }

  const int pb = moe::perm_token_block(d.T, d.E);
  const size_t nb = static_cast<size_t>((d.T + pb - 1) / pb);
  int32_t* block_counts = reinterpret_cast<int32_t*>(base + lw.perm);
  int32_t* block_base =
      reinterpret_cast<int32_t*>(base + lw.perm + align_up(nb * d.E * sizeof(int32_t)));
  e = moe::launch_permute(d, x, topk_idx, 0, d.E, counts, offsets, split, ps, pp, x_perm,
                          block_counts, block_base, s);
  if (e != hipSuccess || d.T == 0) return hip_status(e);  // T == 0: zero counts only

  e = run_ffn(d, d.E, M, d.I, x_perm, offsets, w_gate_up, w_down, h, y_perm, s, base + lw.tail,
              lw.tail_bytes);
  if (e != hipSuccess) return hip_status(e);

  const void* shared_out = nullptr;
  if (d.I_shared > 0) {
    void* s_out = base + lw.s_out;
    e = run_ffn(d, 1, d.T, d.I_shared, x, nullptr, shared_gate_up, shared_down, base + lw.h_sh,
                s_out, s, base + lw.tail, lw.tail_bytes);
    if (e != hipSuccess) return hip_status(e);
    shared_out = s_out;
  }
  return hip_status(
      moe::launch_combine(d, y_perm, pp, topk_w, x, shared_out, 0, d.T, out, s));
}

// ---------------------------------------------------------------------------
// MXFP8 variant of the expert FFN (include/moe_mxfp8.h)
// ---------------------------------------------------------------------------
namespace {

// H in bf16, then its MXFP8 codes and scales.
size_t ffn_mxfp8_ws(int inter, int64_t cap_rows) {
  const size_t hs = static_cast<size_t>(cap_rows) * inter;
  return align_up(hs * 2) + align_up(hs) + align_up(hs / 32);
}

}  // namespace

MOE_API moe_status moe_mxfp8_quantize_rows(int64_t rows, int32_t K, const void* x, void* codes,
                                           void* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return MOE_ERR_INVALID_ARG;
  if (rows >= (int64_t(1) << 40) / K) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_mx_quantize_rows(rows, K, x, codes, scales,
                                                 static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_mxfp8_pack_weights(int32_t n, int32_t K, int32_t N, const void* w,
                                          void* codes, void* scales, void* stream) {
  if (n < 0 || K <= 0 || K % 32 != 0 || N <= 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (w == nullptr || codes == nullptr || scales == nullptr) return MOE_ERR_INVALID_ARG;
  if (static_cast<int64_t>(n) * K * N >= (int64_t(1) << 40) || K / 32 > 65535 ||
      (N + 255) / 256 > 65535)
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_mx_pack_weights(n, K, N, w, codes, scales,
                                                static_cast<hipStream_t>(stream)));
}

MOE_API size_t moe_ffn_mxfp8_workspace_size(const moe_desc* desc, int32_t inter,
                                            int64_t cap_rows) {
  if (check_desc(desc) != MOE_OK || inter <= 0 || cap_rows < 0) return 0;
  return ffn_mxfp8_ws(inter, cap_rows);
}

namespace {
moe_status check_ffn_mxfp8(const moe_desc* desc, int32_t n_experts, int32_t inter,
                           int64_t cap_rows) {
  moe_status st = check_ffn_args(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (desc->act_dtype != MOE_BF16 || desc->D % 128 != 0 || inter % 128 != 0 || y_half(*desc))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}
}  // namespace

MOE_API moe_status moe_expert_gate_up_mxfp8(const moe_desc* desc, int32_t n_experts,
                                            int32_t inter, int64_t cap_rows, const void* xq,
                                            const void* xs, const int32_t* offsets,
                                            const void* w_gu_q, const void* w_gu_s, void* h,
                                            void* stream) {
  moe_status st = check_ffn_mxfp8(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (cap_rows == 0) return MOE_OK;
  if (xq == nullptr || xs == nullptr || offsets == nullptr || w_gu_q == nullptr ||
      w_gu_s == nullptr || h == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_gate_up_mxfp8(n_experts, cap_rows, desc->D, inter, xq, xs,
                                              offsets, w_gu_q, w_gu_s, h,
                                              static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_expert_down_mxfp8(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                         int64_t cap_rows, const void* hq, const void* hs,
                                         const int32_t* offsets, const void* w_d_q,
                                         const void* w_d_s, float* y_perm, void* stream) {
  moe_status st = check_ffn_mxfp8(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (cap_rows == 0) return MOE_OK;
  if (hq == nullptr || hs == nullptr || offsets == nullptr || w_d_q == nullptr ||
      w_d_s == nullptr || y_perm == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_down_mxfp8(n_experts, cap_rows, desc->D, inter, hq, hs, offsets,
                                           w_d_q, w_d_s, y_perm,
                                           static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_expert_ffn_mxfp8(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                        int64_t cap_rows, const void* xq, const void* xs,
                                        const int32_t* offsets, const void* w_gu_q,
                                        const void* w_gu_s, const void* w_d_q,
                                        const void* w_d_s, float* y_perm, void* ws,
                                        size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_mxfp8(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (cap_rows == 0) return MOE_OK;
  if (xq == nullptr || xs == nullptr || offsets == nullptr || w_gu_q == nullptr ||
      w_gu_s == nullptr || w_d_q == nullptr || w_d_s == nullptr || y_perm == nullptr ||
      ws == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_mxfp8_ws(inter, cap_rows)) return MOE_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t hs = static_cast<size_t>(cap_rows) * inter;
  char* base = static_cast<char*>(ws);
  void* h = base;
  void* hq = base + align_up(hs * 2);
  void* hsc = base + align_up(hs * 2) + align_up(hs);
  hipError_t e = moe::launch_gate_up_mxfp8(n_experts, cap_rows, desc->D, inter, xq, xs, offsets,
                                           w_gu_q, w_gu_s, h, s);
  if (e == hipSuccess) e = moe::launch_mx_quantize_rows(cap_rows, inter, h, hq, hsc, s);
  if (e == hipSuccess)
    e = moe::launch_down_mxfp8(n_experts, cap_rows, desc->D, inter, hq, hsc, offsets, w_d_q,
                               w_d_s, y_perm, s);
  return hip_status(e);
}

// ---------------------------------------------------------------------------
// Backward pass (renormalised top-k weights)
// ---------------------------------------------------------------------------
namespace {
moe_status check_bwd_desc(const moe_desc* desc) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  // renormalised top-k weights, stacked expert weights, fp32 expert outputs
  if (desc->norm_topk != 1 || packed(*desc) || y_half(*desc)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline bool is_bf16(const moe_desc& d) { return d.act_dtype == MOE_BF16; }

// dH (fp32 [cap, I]), dG | dU ([cap, 2I]) and H ([cap, I]): bf16 for bf16
// layers, fp32 for fp32 layers (where dG | dU first holds the recomputed
// G | U).
size_t ffn_bwd_ws(const moe_desc& d, int inter, int64_t cap_rows) {
  const size_t r = static_cast<size_t>(cap_rows);
  const size_t s = act_bytes(d);
  return align_up(r * inter * 4) + align_up(r * 2 * inter * s) + align_up(r * inter * s);
}

moe_status check_ffn_bwd(const moe_desc* desc, int32_t n_experts, int32_t inter,
                         int64_t cap_rows) {
  moe_status st = check_ffn_args(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  st = check_bwd_desc(desc);
  if (st != MOE_OK) return st;
  // The bf16 weight-gradient GEMM addresses a segment of rows with 32-bit
  // byte offsets kept below 2^30.
  if (is_bf16(*desc) &&
      cap_rows * static_cast<int64_t>(desc->D > 2 * inter ? desc->D : 2 * inter) * 2 >=
          (int64_t(1) << 30))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// fp32 layers: G | U recomputed into dgu, the SiLU-gate adjoint in place.
hipError_t run_gate_up_bwd_f32(const moe_desc& d, int n, int inter, int64_t cap,
                               const void* x_perm, const int32_t* offsets, const void* w_gate_up,
                               const float* dh, float* dgu, float* h, hipStream_t s) {
  hipError_t e = moe::launch_rows_gemm_f32(
      n, cap, static_cast<const float*>(x_perm), offsets, static_cast<const float*>(w_gate_up),
      static_cast<int64_t>(d.D) * 2 * inter, 2 * inter, 1, dgu, d.D, 2 * inter, s);
  if (e == hipSuccess) e = moe::launch_swiglu_bwd_f32(cap, inter, dh, dgu, h, s);
  return e;
}

hipError_t run_ffn_bwd_f32(const moe_desc& d, int n, int inter, int64_t cap, const void* x_perm,
                           const int32_t* offsets, const void* w_gate_up, const void* w_down,
                           const void* dy_perm, float* dx_perm, float* dw_gate_up,
                           float* dw_down, void* ws, hipStream_t s) {
  const size_t r = static_cast<size_t>(cap);
  char* base = static_cast<char*>(ws);
  float* dh = reinterpret_cast<float*>(base);
  float* dgu = reinterpret_cast<float*>(base + align_up(r * inter * 4));
  float* h = reinterpret_cast<float*>(base + align_up(r * inter * 4) + align_up(r * 2 * inter * 4));
  const float* dy = static_cast<const float*>(dy_perm);
  const float* x = static_cast<const float*>(x_perm);
  // dH[r, i] = sum_d dy[r, d] Wd[e][i][d]
  hipError_t e = moe::launch_rows_gemm_f32(n, cap, dy, offsets, static_cast<const float*>(w_down),
                                           static_cast<int64_t>(inter) * d.D, 1, d.D, dh, d.D,
                                           inter, s);
  if (e == hipSuccess)
    e = run_gate_up_bwd_f32(d, n, inter, cap, x_perm, offsets, w_gate_up, dh, dgu, h, s);
  // dx[r, d] = sum_c dGU[r, c] Wgu[e][d][c]
  if (e == hipSuccess && dx_perm != nullptr)
    e = moe::launch_rows_gemm_f32(n, cap, dgu, offsets, static_cast<const float*>(w_gate_up),
                                  static_cast<int64_t>(d.D) * 2 * inter, 1, 2 * inter, dx_perm,
                                  2 * inter, d.D, s);
  if (e == hipSuccess)
    e = moe::launch_contract_gemm_f32(n, cap, h, inter, dy, d.D, offsets, dw_down, s);
  if (e == hipSuccess)
    e = moe::launch_contract_gemm_f32(n, cap, x, d.D, dgu, 2 * inter, offsets, dw_gate_up, s);
  return e;
}

// gu_saved: G | U of the training forward (bf16 layers), else NULL (G | U
// recomputed).
hipError_t run_ffn_bwd(const moe_desc& d, int n, int inter, int64_t cap, const void* x_perm,
                       const int32_t* offsets, const void* w_gate_up, const void* w_down,
                       const void* dy_perm, const float* gu_saved, float* dx_perm,
                       float* dw_gate_up, float* dw_down, void* ws, hipStream_t s) {
  if (!is_bf16(d))
    return run_ffn_bwd_f32(d, n, inter, cap, x_perm, offsets, w_gate_up, w_down, dy_perm,
                           dx_perm, dw_gate_up, dw_down, ws, s);
  const size_t r = static_cast<size_t>(cap);
  char* base = static_cast<char*>(ws);
  float* dh = reinterpret_cast<float*>(base);
  void* dgu = base + align_up(r * inter * 4);
  void* h = base + align_up(r * inter * 4) + align_up(r * 2 * inter * 2);
  hipError_t e;
  if (gu_saved != nullptr) {
    e = moe::launch_dh_swiglu_saved(n, cap, d.D, inter, dy_perm, offsets, w_down, gu_saved, dgu,
                                    h, s);
  } else {
    e = moe::launch_dh_bwd(n, cap, d.D, inter, dy_perm, offsets, w_down, dh, s);
    if (e == hipSuccess)
      e = moe::launch_gate_up_bwd_bf16(n, cap, d.D, inter, x_perm, offsets, w_gate_up, dh, dgu,
                                       h, s);
  }
  if (e == hipSuccess && dx_perm != nullptr)
    e = moe::launch_dx_perm_bwd(n, cap, d.D, inter, dgu, offsets, w_gate_up, dx_perm, s);
  if (e == hipSuccess)
    e = moe::launch_wgrad_bf16(n, cap, h, inter, dy_perm, d.D, offsets, dw_down, s);
  if (e == hipSuccess)
    e = moe::launch_wgrad_bf16(n, cap, x_perm, d.D, dgu, 2 * inter, offsets, dw_gate_up, s);
  return e;
}

size_t router_bwd_ws(const moe_desc& d, int64_t cap_rows) {
  return align_up(moe::router_bwd_partial_floats(cap_rows, d.E, d.D) * sizeof(float));
}

// Layer backward workspace: dy_perm, dlogit, dl_perm, dx_perm, the FFN
// backward's, the router's, and for a shared expert dx_shared and its FFN
// backward's.
struct BwdWs {
  size_t dy, dl, dlp, dxp, ffn, router, dxs, ffn_sh, total;
};

BwdWs bwd_ws(const moe_desc& d) {
  BwdWs w{};
  const int64_t M = static_cast<int64_t>(d.T) * d.top_k;
  const size_t m = static_cast<size_t>(M), t = static_cast<size_t>(d.T);
  size_t o = 0;
  w.dy = o;      o += align_up(m * d.D * act_bytes(d));
  w.dl = o;      o += align_up(t * d.top_k * 4);
  w.dlp = o;     o += align_up(m * 4);
  w.dxp = o;     o += align_up(m * d.D * 4);
  w.ffn = o;     o += ffn_bwd_ws(d, d.I, M);
  w.router = o;  o += router_bwd_ws(d, M);
  w.dxs = o;     o += d.I_shared > 0 ? align_up(t * d.D * 4) : 0;
  w.ffn_sh = o;  o += d.I_shared > 0 ? ffn_bwd_ws(d, d.I_shared, d.T) : 0;
  w.total = o;
  return w;
}
}  // namespace

MOE_API moe_status moe_combine_backward(const moe_desc* desc, const void* dout,
                                        const float* y_perm, const int32_t* pos,
                                        const float* topk_w, void* dy_perm, float* dtopk_w,
                                        float* dlogit, float* dl_perm, void* stream) {
  moe_status st = check_bwd_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (dout == nullptr || y_perm == nullptr || pos == nullptr || topk_w == nullptr ||
      dy_perm == nullptr || dlogit == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine_bwd(is_bf16(*desc), desc->T, desc->D, desc->top_k, dout,
                                            y_perm, pos,
                                            topk_w, dy_perm, dtopk_w, dlogit, dl_perm,
                                            static_cast<hipStream_t>(stream)));
}

MOE_API size_t moe_ffn_backward_workspace_size(const moe_desc* desc, int32_t inter,
                                               int64_t cap_rows) {
  if (check_desc(desc) != MOE_OK || inter <= 0 || cap_rows < 0) return 0;
  return ffn_bwd_ws(*desc, inter, cap_rows);
}

MOE_API moe_status moe_expert_ffn_backward(const moe_desc* desc, int32_t n_experts, int32_t inter,
                                           int64_t cap_rows, const void* x_perm,
                                           const int32_t* offsets, const void* w_gate_up,
                                           const void* w_down, const void* dy_perm,
                                           const float* gu_saved, float* dx_perm,
                                           float* dw_gate_up, float* dw_down, void* ws,
                                           size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_bwd(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (gu_saved != nullptr && !is_bf16(*desc)) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr && n_experts != 1) return MOE_ERR_INVALID_ARG;
  if (w_gate_up == nullptr || w_down == nullptr || dw_gate_up == nullptr || dw_down == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (cap_rows > 0 && (x_perm == nullptr || dy_perm == nullptr || ws == nullptr))
    return MOE_ERR_INVALID_ARG;
  if (cap_rows > 0 && ws_bytes < ffn_bwd_ws(*desc, inter, cap_rows)) return MOE_ERR_WORKSPACE;
  return hip_status(run_ffn_bwd(*desc, n_experts, inter, cap_rows, x_perm, offsets, w_gate_up,
                                w_down, dy_perm, gu_saved, dx_perm, dw_gate_up, dw_down, ws,
                                static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_expert_gate_up_backward(const moe_desc* desc, int32_t n_experts,
                                               int32_t inter, int64_t cap_rows,
                                               const void* x_perm, const int32_t* offsets,
                                               const void* w_gate_up, const float* dh, void* dgu,
                                               void* h, void* stream) {
  moe_status st = check_ffn_bwd(desc, n_experts, inter, cap_rows);
  if (st != MOE_OK) return st;
  if (offsets == nullptr && n_experts != 1) return MOE_ERR_INVALID_ARG;
  if (cap_rows == 0) return MOE_OK;
  if (x_perm == nullptr || w_gate_up == nullptr || dh == nullptr || dgu == nullptr ||
      h == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!is_bf16(*desc))
    return hip_status(run_gate_up_bwd_f32(*desc, n_experts, inter, cap_rows, x_perm, offsets,
                                          w_gate_up, dh, static_cast<float*>(dgu),
                                          static_cast<float*>(h),
                                          static_cast<hipStream_t>(stream)));
  return hip_status(moe::launch_gate_up_bwd_bf16(n_experts, cap_rows, desc->D, inter, x_perm,
                                                 offsets, w_gate_up, dh, dgu, h,
                                                 static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_expert_weight_grad(const moe_desc* desc, int32_t n_experts,
                                          int64_t cap_rows, const void* a, int32_t P,
                                          const void* b, int32_t Q, const int32_t* offsets,
                                          float* c, void* stream) {
  moe_status st = check_bwd_desc(desc);
  if (st != MOE_OK) return st;
  if (n_experts < 1 || cap_rows < 0 || P <= 0 || Q <= 0) return MOE_ERR_INVALID_ARG;
  if (offsets == nullptr && n_experts != 1) return MOE_ERR_INVALID_ARG;
  if (n_experts > MOE_MAX_EXPERTS || P % 64 != 0 || Q % 64 != 0 || cap_rows > INT_MAX ||
      (is_bf16(*desc) &&
       cap_rows * static_cast<int64_t>(P > Q ? P : Q) * 2 >= (int64_t(1) << 30)) ||
      // 32-bit row offsets inside a K step of 32 rows
      P > (1 << 24) || Q > (1 << 24) ||
      // one workgroup per 128 x 256 tile, rounded up to 8 per expert
      static_cast<int64_t>(n_experts) *
              ((static_cast<int64_t>(P) + 127) / 128 * ((static_cast<int64_t>(Q) + 255) / 256) +
               7) > INT_MAX)
    return MOE_ERR_UNSUPPORTED;
  if (c == nullptr || (cap_rows > 0 && (a == nullptr || b == nullptr))) return MOE_ERR_INVALID_ARG;
  if (!is_bf16(*desc))
    return hip_status(moe::launch_contract_gemm_f32(
        n_experts, cap_rows, static_cast<const float*>(a), P, static_cast<const float*>(b), Q,
        offsets, c, static_cast<hipStream_t>(stream)));
  return hip_status(moe::launch_wgrad_bf16(n_experts, cap_rows, a, P, b, Q, offsets, c,
                                           static_cast<hipStream_t>(stream)));
}

MOE_API size_t moe_router_backward_workspace_size(const moe_desc* desc, int64_t cap_rows) {
  if (check_desc(desc) != MOE_OK || cap_rows < 0) return 0;
  return router_bwd_ws(*desc, cap_rows);
}

MOE_API moe_status moe_router_backward(const moe_desc* desc, int64_t cap_rows, const void* x_perm,
                                       const int32_t* offsets, const float* dl_perm,
                                       float* dw_router, void* ws, size_t ws_bytes,
                                       void* stream) {
  moe_status st = check_bwd_desc(desc);
  if (st != MOE_OK) return st;
  if (cap_rows < 0) return MOE_ERR_INVALID_ARG;
  if (cap_rows > INT_MAX) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr || dw_router == nullptr || ws == nullptr) return MOE_ERR_INVALID_ARG;
  if (cap_rows > 0 && (x_perm == nullptr || dl_perm == nullptr)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < router_bwd_ws(*desc, cap_rows)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_router_bwd(is_bf16(*desc), cap_rows, desc->D, desc->E, x_perm,
                                           offsets, dl_perm,
                                           static_cast<float*>(ws), dw_router,
                                           static_cast<hipStream_t>(stream)));
}

MOE_API moe_status moe_input_backward(const moe_desc* desc, const float* dx_perm,
                                      const int32_t* pos, const int32_t* topk_idx,
                                      const float* dlogit, const float* w_router,
                                      const float* dx_shared, const void* dout, void* dx,
                                      void* stream) {
  moe_status st = check_bwd_desc(desc);
  if (st != MOE_OK) return st;
  if (desc->T == 0) return MOE_OK;
  if (dx_perm == nullptr || pos == nullptr || dx == nullptr) return MOE_ERR_INVALID_ARG;
  if (dlogit != nullptr && (topk_idx == nullptr || w_router == nullptr))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_input_bwd(is_bf16(*desc), desc->T, desc->D, desc->top_k, dx_perm,
                                          pos, topk_idx,
                                          dlogit, w_router, dx_shared, dout, dx,
                                          static_cast<hipStream_t>(stream)));
}

MOE_API size_t moe_backward_workspace_size(const moe_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return bwd_ws(*desc).total;
}

MOE_API moe_status moe_layer_backward(const moe_desc* desc, const void* x, const float* w_router,
                                      const void* w_gate_up, const void* w_down,
                                      const void* shared_gate_up, const void* shared_down,
                                      const int32_t* topk_idx, const float* topk_w,
                                      const int32_t* offsets, const int32_t* pos,
                                      const void* x_perm, const float* y_perm,
                                      const float* gu_saved, const float* gu_shared_saved,
                                      const void* dout, void* dx, float* dw_router,
                                      float* dw_gate_up,
                                      float* dw_down, float* dw_shared_gate_up,
                                      float* dw_shared_down, void* ws, size_t ws_bytes,
                                      void* stream) {
  moe_status st = check_bwd_desc(desc);
  if (st != MOE_OK) return st;
  const int64_t M = static_cast<int64_t>(desc->T) * desc->top_k;
  st = check_ffn_bwd(desc, desc->E, desc->I, M);
  if (st != MOE_OK) return st;
  if (desc->I_shared > 0) {
    st = check_ffn_bwd(desc, 1, desc->I_shared, desc->T);
    if (st != MOE_OK) return st;
    if (shared_gate_up == nullptr || shared_down == nullptr || dw_shared_gate_up == nullptr ||
        dw_shared_down == nullptr)
      return MOE_ERR_INVALID_ARG;
  }
  if (w_router == nullptr || w_gate_up == nullptr || w_down == nullptr || offsets == nullptr ||
      dw_router == nullptr || dw_gate_up == nullptr || dw_down == nullptr || ws == nullptr)
    return MOE_ERR_INVALID_ARG;
  if ((gu_saved != nullptr || gu_shared_saved != nullptr) && !is_bf16(*desc))
    return MOE_ERR_UNSUPPORTED;
  if (desc->T > 0 && (x == nullptr || topk_idx == nullptr || topk_w == nullptr ||
                      pos == nullptr || x_perm == nullptr || y_perm == nullptr ||
                      dout == nullptr || dx == nullptr))
    return MOE_ERR_INVALID_ARG;
  const BwdWs w = bwd_ws(*desc);
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  void* dy = base + w.dy;
  float* dl = reinterpret_cast<float*>(base + w.dl);
  float* dlp = reinterpret_cast<float*>(base + w.dlp);
  float* dxp = reinterpret_cast<float*>(base + w.dxp);
  float* dxs = desc->I_shared > 0 ? reinterpret_cast<float*>(base + w.dxs) : nullptr;
  const bool bf = is_bf16(*desc);
  hipError_t e = moe::launch_combine_bwd(bf, desc->T, desc->D, desc->top_k, dout, y_perm, pos,
                                         topk_w,
                                         dy, nullptr, dl, dlp, s);
  if (e == hipSuccess)
    e = run_ffn_bwd(*desc, desc->E, desc->I, M, x_perm, offsets, w_gate_up, w_down, dy, gu_saved,
                    dxp, dw_gate_up, dw_down, base + w.ffn, s);
  if (e == hipSuccess && dxs != nullptr)
    e = run_ffn_bwd(*desc, 1, desc->I_shared, desc->T, x, nullptr, shared_gate_up, shared_down,
                    dout, gu_shared_saved, dxs, dw_shared_gate_up, dw_shared_down,
                    base + w.ffn_sh, s);
  if (e == hipSuccess)
    e = moe::launch_router_bwd(bf, M, desc->D, desc->E, x_perm, offsets, dlp,
                               reinterpret_cast<float*>(base + w.router), dw_router, s);
  if (e == hipSuccess)
    e = moe::launch_input_bwd(bf, desc->T, desc->D, desc->top_k, dxp, pos, topk_idx, dl, w_router,
                              dxs, dout, dx, s);
  return hip_status(e);
}

