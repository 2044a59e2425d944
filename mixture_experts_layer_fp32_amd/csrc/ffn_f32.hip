// Grouped expert FFN in fp32 (activations and weights fp32, fp32 accumulate).
//
// Same computation as the bf16 path (page "Expert Parallel (EP)",
// Communication Pattern stage 3; page "Worked Example", Step 3):
//   H = SiLU(X Wg) * (X Wu),  Y = H Wd  per expert segment.
// A 256-thread workgroup computes 64 rows x 64 output columns with K steps
// of 16 staged in LDS; each thread owns a 4 x 4 block (two of them, gate and
// up, for the gated GEMM). fp32 dense work on this chip runs at the same peak
// on the vector ALUs as on the fp32 matrix instructions, and this path serves
// small fp32 layers, so it stays on the vector ALUs.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 64, BN = 64, BK = 16;

template <bool GATED>
__global__ __launch_bounds__(kThreads) void ffn_gemm_f32(const float* __restrict__ A,
                                                         const int32_t* __restrict__ offsets,
                                                         int n_experts, int64_t cap_rows,
                                                         const float* __restrict__ W,
                                                         float* __restrict__ C, int K, int N_out) {
  constexpr int BNB = GATED ? 2 * BN : BN;
  __shared__ __attribute__((aligned(16))) float As[BK][BM];
  __shared__ __attribute__((aligned(16))) float Bs[BK][BNB];
  __shared__ int s_tile[3];
  const int tid = threadIdx.x;
  if (tid < 64) {
    TileRows tr = find_tile_rows(offsets, n_experts, cap_rows, blockIdx.x, BM);
    if (tid == 0) {
      s_tile[0] = tr.expert;
      s_tile[1] = tr.row_begin;
      s_tile[2] = tr.row_end;
    }
  }
  __syncthreads();
  const int expert = s_tile[0];
  if (expert < 0) return;
  const int row_begin = s_tile[1], row_end = s_tile[2];
  const int n0 = blockIdx.y * BN;
  const int ldw = GATED ? 2 * N_out : N_out;
  const float* Wexp = W + static_cast<int64_t>(expert) * K * ldw;

  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4], accu[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = accu[i][j] = 0.f;

  // A loader: row tid/4, k chunk (tid%4)*4.
  const int la_row = tid >> 2, la_k = (tid & 3) * 4;
  const bool la_ok = row_begin + la_row < row_end;
  const float* la_ptr = A + static_cast<int64_t>(la_ok ? row_begin + la_row : row_begin) * K + la_k;
  // B loader: k row tid/16, columns (tid%16)*4 of the gate (and up) block.
  const int lb_k = tid >> 4, lb_c = (tid & 15) * 4;
  const bool lb_ok = n0 + lb_c < N_out;

  for (int k0 = 0; k0 < K; k0 += BK) {
    const float4 av = la_ok ? *reinterpret_cast<const float4*>(la_ptr + k0) : make_float4(0, 0, 0, 0);
    const float* brow = Wexp + static_cast<int64_t>(k0 + lb_k) * ldw;
    const float4 bv = lb_ok ? *reinterpret_cast<const float4*>(brow + n0 + lb_c) : make_float4(0, 0, 0, 0);
    float4 buv = make_float4(0, 0, 0, 0);
    if (GATED && lb_ok) buv = *reinterpret_cast<const float4*>(brow + N_out + n0 + lb_c);
    __syncthreads();
    As[la_k + 0][la_row] = av.x;
    As[la_k + 1][la_row] = av.y;
    As[la_k + 2][la_row] = av.z;
    As[la_k + 3][la_row] = av.w;
    *reinterpret_cast<float4*>(&Bs[lb_k][lb_c]) = bv;
    if (GATED) *reinterpret_cast<float4*>(&Bs[lb_k][BN + lb_c]) = buv;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
      const float ar[4] = {a.x, a.y, a.z, a.w};
      const float br[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
      if (GATED) {
        const float4 u = *reinterpret_cast<const float4*>(&Bs[kk][BN + tx * 4]);
        const float ur[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) accu[i][j] = fmaf(ar[i], ur[j], accu[i][j]);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row_begin + ty * 4 + i;
    if (row >= row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N_out) continue;
      float v = acc[i][j];
      if (GATED) v = v / (1.f + expf(-v)) * accu[i][j];
      C[static_cast<int64_t>(row) * N_out + col] = v;
    }
  }
}

}  // namespace

namespace {
int64_t m_tiles(int64_t cap_rows, const int32_t* offsets, int n_experts) {
  return (cap_rows + BM - 1) / BM + (offsets ? n_experts : 0);
}
}  // namespace

hipError_t launch_gate_up_f32(int n_experts, int64_t cap_rows, int D, int inter,
                              const void* x_perm, const int32_t* offsets, const void* w_gate_up,
                              void* h, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(m_tiles(cap_rows, offsets, n_experts)),
               (inter + BN - 1) / BN);
  ffn_gemm_f32<true><<<g, kThreads, 0, s>>>(static_cast<const float*>(x_perm), offsets,
                                            n_experts, cap_rows,
                                            static_cast<const float*>(w_gate_up),
                                            static_cast<float*>(h), D, inter);
  return hipGetLastError();
}

hipError_t launch_down_f32(int n_experts, int64_t cap_rows, int D, int inter, const void* h,
                           const int32_t* offsets, const void* w_down, void* y, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(m_tiles(cap_rows, offsets, n_experts)), (D + BN - 1) / BN);
  ffn_gemm_f32<false><<<g, kThreads, 0, s>>>(static_cast<const float*>(h), offsets, n_experts,
                                             cap_rows, static_cast<const float*>(w_down),
                                             static_cast<float*>(y), inter, D);
  return hipGetLastError();
}

}  // namespace moe
