// Internal declarations shared by the HIP sources of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- bf16 helpers (bf16 is carried as raw 16-bit words) -------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float load_act(const float* p) { return *p; }
__device__ __forceinline__ float load_act(const uint16_t* p) { return bf16_to_f32(*p); }

// ---- grouped-GEMM tile lookup --------------------------------------------
// Expert segments are [offsets[e], offsets[e+1]); each is cut into tiles of
// `bm` rows. Tile `tile` (a global index over all experts, in expert order)
// maps to expert e and rows [row_begin, row_end). Computed by one wave from
// the device-resident offsets, so no host round trip is needed.
struct TileRows {
  int expert;     // -1: this tile index is past the last tile
  int row_begin;  // first row of the tile
  int row_end;    // one past the last row of the expert's segment
};

__device__ __forceinline__ TileRows find_tile_rows(const int* __restrict__ offsets,
                                                   int n_experts, int64_t cap_rows,
                                                   int tile, int bm) {
  TileRows r{-1, 0, 0};
  if (offsets == nullptr) {  // one expert owning every row
    int64_t rb = static_cast<int64_t>(tile) * bm;
    if (rb < cap_rows) r = TileRows{0, static_cast<int>(rb), static_cast<int>(cap_rows)};
    return r;
  }
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int e0 = 0; e0 < n_experts; e0 += 64) {
    const int e = e0 + lane;
    int beg = 0, cnt = 0;
    if (e < n_experts) {
      beg = offsets[e];
      cnt = max(offsets[e + 1] - beg, 0);
    }
    const int tiles = (cnt + bm - 1) / bm;
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int excl = incl - tiles;
    const bool hit = tiles > 0 && tile >= base + excl && tile < base + incl;
    const unsigned long long m = __ballot(hit);
    if (m) {
      const int src = __ffsll(static_cast<long long>(m)) - 1;
      const int hb = __shfl(beg, src, 64);
      const int hc = __shfl(cnt, src, 64);
      const int hx = __shfl(excl, src, 64);
      r.expert = e0 + src;
      r.row_begin = hb + (tile - base - hx) * bm;
      // Rows never extend past the buffers' capacity, whatever the offsets say.
      r.row_end = static_cast<int>(min(static_cast<int64_t>(hb + hc), cap_rows));
      if (r.row_begin < 0 || r.row_begin >= r.row_end) r.expert = -1;
      return r;
    }
    base += __shfl(incl, 63, 64);
  }
  return r;
}

// ---- launchers (each returns the launch's hipError_t) ---------------------
// bf16 activations with the fp32 router: approximate bf16-split logits, a
// certified top-k and exact fp64 recompute of the uncertain candidates; ws
// holds route_ws_bytes(d) bytes. fp32 activations: the fp64 router (ws unused).
size_t route_ws_bytes(const moe_desc& d);
hipError_t launch_route(const moe_desc& d, const void* x, const float* w_router,
                        const float* bias, float* logits, float* probs, int32_t* topk_idx,
                        float* topk_w, void* ws, hipStream_t s);
// router_dtype MOE_F32 / MOE_BF16 / MOE_F16: gate weight and logits in that
// dtype (logits the correctly rounded dot product).
hipError_t launch_route_typed(const moe_desc& d, int router_dtype, const void* x,
                              const void* w_router, const float* bias, void* logits, float* probs,
                              int32_t* topk_idx, float* topk_w, hipStream_t s);

// Permute: counts of tokens are taken per block of kPermBlock tokens; blocks
// grow until blocks x experts <= kPermMaxBlockCounts (the scan holds them in
// LDS), so the permute's scratch never exceeds 2 kPermMaxBlockCounts ints.
constexpr int kPermBlock = 256;
constexpr int kPermMaxBlockCounts = 12288;
int perm_token_block(int T, int n);  // tokens per count block (a multiple of kPermBlock)
hipError_t launch_permute(const moe_desc& d, const void* x, const int32_t* topk_idx,
                          int e_begin, int e_end, int32_t* counts, int32_t* offsets,
                          int32_t* split, int32_t* perm_src, int32_t* pos, void* x_perm,
                          int32_t* block_counts, int32_t* block_base, hipStream_t s);

// Grouped SiLU-gated FFN. gate_up: h = SiLU(x Wg) * (x Wu); down: y = h Wd.
// offsets == nullptr: one expert owning all cap_rows rows. bf16 layers keep h
// in fp16; y is fp32. w_ptrs (device array of n_experts pointers) replaces the
// stacked weight when not null (one buffer per expert, same per-expert layout).
// packed: the weights are in the operand order launch_pack_weights writes
// (down_proj in fp16) instead of stacked [n][K][N].
// tail_ws, tail_bytes: the split-K part buffer (packed weights only), as for
// the down GEMM below.
hipError_t launch_gate_up_bf16(int n_experts, int64_t cap_rows, int D, int inter,
                               const void* x_perm, const int32_t* offsets, const void* w_gate_up,
                               void* h, hipStream_t s, const void* const* w_ptrs = nullptr,
                               bool packed = false, void* tail_ws = nullptr,
                               size_t tail_bytes = 0);
// y_half: y written in fp16 (saturating at +-65504) instead of fp32.
hipError_t launch_down_bf16(int n_experts, int64_t cap_rows, int D, int inter, const void* h,
                            const int32_t* offsets, const void* w_down, void* y, hipStream_t s,
                            const void* const* w_ptrs = nullptr, bool packed = false,
                            bool y_half = false, void* tail_ws = nullptr, size_t tail_bytes = 0);
// The split-K tail: with a part buffer (tail_ws, tail_bytes) the tiles of the
// last, partial round of wide tiles are cut along K, one part of
// kDownPartBytes per unit, followed by a header (tail size, part count, each
// tail tile's place in the output), and summed by a second launch. Bytes
// that always suffice for cap_rows rows, n_experts experts and D output
// columns (down GEMM) or inter H columns (gated GEMM).
constexpr size_t kDownPartBytes = 256 * 1024;
constexpr int64_t kMaxTailUnits = 256;
constexpr size_t kTailHeaderBytes = 16 * (kMaxTailUnits + 1);
size_t down_tail_bytes(int64_t cap_rows, int n_experts, int D);
size_t gate_up_tail_bytes(int64_t cap_rows, int n_experts, int inter);
// [n][K][N] 16-bit weights -> packed operand order (to_f16: bf16 -> fp16).
hipError_t launch_pack_weights(int n, int K, int N, bool to_f16, const void* w, void* out,
                               hipStream_t s);
// Tile shape the bf16 grouped GEMMs take (host arithmetic; gemm 0 = gate_up,
// 1 = down): rows and product columns per workgroup tile.
void ffn_tile_shape_bf16(int n_experts, int64_t cap_rows, int D, int inter, bool has_offsets,
                         int gemm, int* rows, int* cols);
hipError_t launch_gate_up_f32(int n_experts, int64_t cap_rows, int D, int inter,
                              const void* x_perm, const int32_t* offsets, const void* w_gate_up,
                              void* h, hipStream_t s);
hipError_t launch_down_f32(int n_experts, int64_t cap_rows, int D, int inter, const void* h,
                           const int32_t* offsets, const void* w_down, void* y, hipStream_t s);

// MXFP8 expert FFN (ffn_mxfp8.hip, mxfp8_quant.hip).
hipError_t launch_mx_quantize_rows(int64_t rows, int K, const void* x, void* codes, void* scales,
                                   hipStream_t s);
hipError_t launch_mx_pack_weights(int n, int K, int N, const void* w, void* codes, void* scales,
                                  hipStream_t s);
hipError_t launch_gate_up_mxfp8(int n_experts, int64_t cap_rows, int D, int inter,
                                const void* xq, const void* xs, const int32_t* offsets,
                                const void* wq, const void* wsc, void* h, hipStream_t s);
hipError_t launch_down_mxfp8(int n_experts, int64_t cap_rows, int D, int inter, const void* hq,
                             const void* hs, const int32_t* offsets, const void* wq,
                             const void* wsc, void* y, hipStream_t s);
// Backward pass (ffn_bwd.hip, backward.hip; bf16 layers).
// Training forward GEMM 1: h as launch_gate_up_bf16, and G | U saved in fp32
// to gu [cap, 2 inter].
hipError_t launch_gate_up_save_bf16(int n_experts, int64_t cap_rows, int D, int inter,
                                    const void* x_perm, const int32_t* offsets,
                                    const void* w_gate_up, void* h, float* gu, hipStream_t s);
// dH = dy W_down^T with the SiLU-gate adjoint from the saved G | U (fp32):
// dgu = dG | dU [cap, 2 inter], h = SiLU(G) U [cap, inter] (bf16).
hipError_t launch_dh_swiglu_saved(int n_experts, int64_t cap_rows, int D, int inter,
                                  const void* dy_perm, const int32_t* offsets,
                                  const void* w_down, const float* gu, void* dgu, void* h,
                                  hipStream_t s);
// dH = dy W_down^T, fp32 [cap, inter].
hipError_t launch_dh_bwd(int n_experts, int64_t cap_rows, int D, int inter, const void* dy_perm,
                         const int32_t* offsets, const void* w_down, float* dh, hipStream_t s);
// G | U = x_perm W_gate_up recomputed in the accumulators; the epilogue reads
// dH and writes dgu = dG | dU [cap, 2 inter] and h = SiLU(G) U [cap, inter]
// (bf16).
hipError_t launch_gate_up_bwd_bf16(int n_experts, int64_t cap_rows, int D, int inter,
                                   const void* x_perm, const int32_t* offsets,
                                   const void* w_gate_up, const float* dh, void* dgu, void* h,
                                   hipStream_t s);
// dx_perm = dgu W_gate_up^T (fp32).
hipError_t launch_dx_perm_bwd(int n_experts, int64_t cap_rows, int D, int inter, const void* dgu,
                              const int32_t* offsets, const void* w_gate_up, float* dx_perm,
                              hipStream_t s);
// c[e] = a_e^T b_e over each expert's rows: a [cap, P], b [cap, Q] bf16,
// c [n, P, Q] fp32 (zero for an expert without rows).
hipError_t launch_wgrad_bf16(int n_experts, int64_t cap_rows, const void* a, int P, const void* b,
                             int Q, const int32_t* offsets, float* c, hipStream_t s);
// bf16: activations (dout, dy_perm, x_perm, dx) in bf16, else fp32.
hipError_t launch_combine_bwd(bool bf16, int T, int D, int k, const void* dout,
                              const float* y_perm, const int32_t* pos, const float* topk_w,
                              void* dy_perm, float* dtopk_w, float* dlogit, float* dl_perm,
                              hipStream_t s);
hipError_t launch_input_bwd(bool bf16, int T, int D, int k, const float* dx_perm,
                            const int32_t* pos, const int32_t* topk_idx, const float* dlogit,
                            const float* w_router, const float* dx_shared, const void* dout,
                            void* dx, hipStream_t s);
size_t router_bwd_partial_floats(int64_t cap_rows, int E, int D);
hipError_t launch_router_bwd(bool bf16, int64_t cap_rows, int D, int E, const void* x_perm,
                             const int32_t* offsets, const float* dl_perm, float* partial,
                             float* dw_router, hipStream_t s);
// fp32 layers (bwd_f32.hip): C[r, n] = sum_k A[r, k] W[e*w_es + k*w_sk + n*w_sn]
// over each expert's rows; C_e = A_e^T B_e over each expert's rows; the
// SiLU-gate adjoint in place over G | U.
hipError_t launch_rows_gemm_f32(int n_experts, int64_t cap_rows, const float* a,
                                const int32_t* offsets, const float* w, int64_t w_es,
                                int64_t w_sk, int64_t w_sn, float* c, int K, int N,
                                hipStream_t s);
hipError_t launch_contract_gemm_f32(int n_experts, int64_t cap_rows, const float* a, int P,
                                    const float* b, int Q, const int32_t* offsets, float* c,
                                    hipStream_t s);
hipError_t launch_swiglu_bwd_f32(int64_t rows, int inter, const float* dh, float* gu, float* h,
                                 hipStream_t s);

// y_perm and shared_out are fp16 when d.expert_out_dtype is MOE_F16, else fp32.
hipError_t launch_combine(const moe_desc& d, const void* y_perm, const int32_t* pos,
                          const float* topk_w, const void* residual, const void* shared_out,
                          int res_begin, int res_rows, void* out, hipStream_t s);

}  // namespace moe
