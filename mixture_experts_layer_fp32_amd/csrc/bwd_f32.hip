// Backward pass of the expert FFN for fp32 layers (fp32 throughout, on the
// vector ALUs like the fp32 forward: these layers are small).
//
// Gradients per expert segment (page "Expert Parallel (EP)", Communication
// Pattern stage 3; page "Worked Example", Step 3), as for bf16 layers:
//   dH = dY Wd^T;  G | U = X Wgu;  dG = dH U SiLU'(G), dU = dH SiLU(G),
//   H = SiLU(G) U;  dX = [dG | dU] Wgu^T;  dWd = H^T dY;  dWgu = X^T [dG | dU].
// Two tiled kernels cover the products: rows_gemm (C = A op(B) over each
// expert's rows, B = W_e read with arbitrary strides) and contract_gemm
// (C_e = A_e^T B_e, the contraction over each expert's rows); swiglu_bwd
// forms dG | dU and H elementwise (in place over G | U).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 64, BN = 64, BK = 16;

// C[r, n] = sum_k A[r, k] B_e(k, n) for the rows r of each expert segment,
// B_e(k, n) = W[e * w_es + k * w_sk + n * w_sn]. A is [cap, K] row-major,
// C [cap, N] row-major. Grid: (row tiles over all segments, N / BN).
__global__ __launch_bounds__(kThreads) void rows_gemm(
    const float* __restrict__ A, const int32_t* __restrict__ offsets, int n_experts,
    int64_t cap_rows, const float* __restrict__ W, int64_t w_es, int64_t w_sk, int64_t w_sn,
    float* __restrict__ C, int K, int N) {
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs[BK][BN + 1];
  __shared__ int s_tile[3];
  const int tid = threadIdx.x;
  if (tid < 64) {
    const TileRows tr = find_tile_rows(offsets, n_experts, cap_rows, blockIdx.x, BM);
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
  const float* We = W + static_cast<int64_t>(expert) * w_es;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int i = tid; i < BK * BM; i += kThreads) {
      const int r = i / BK, k = i % BK;  // consecutive threads along k (contiguous in A)
      const int row = row_begin + r;
      As[k][r] = row < row_end && k0 + k < K ? A[static_cast<int64_t>(row) * K + k0 + k] : 0.f;
    }
    for (int i = tid; i < BK * BN; i += kThreads) {
      const int k = i / BN, n = i % BN;
      Bs[k][n] = k0 + k < K && n0 + n < N ? We[(k0 + k) * w_sk + (n0 + n) * w_sn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[k][ty * 4 + i];
        b[i] = Bs[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row_begin + ty * 4 + i;
    if (row >= row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) C[static_cast<int64_t>(row) * N + n] = acc[i][j];
    }
  }
}

// C_e[p, q] = sum over the rows m of expert e of A[m, p] B[m, q]; A [cap, P],
// B [cap, Q], C [n, P, Q]. Grid: (Q / BN, P / BM, n_experts).
__global__ __launch_bounds__(kThreads) void contract_gemm(
    const float* __restrict__ A, int P, const float* __restrict__ B, int Q,
    const int32_t* __restrict__ offsets, int64_t cap_rows, float* __restrict__ C) {
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs[BK][BN + 1];
  const int e = blockIdx.z;
  int64_t beg = 0, end = cap_rows;
  if (offsets) {
    beg = min(max(static_cast<int64_t>(offsets[e]), int64_t(0)), cap_rows);
    end = min(max(static_cast<int64_t>(offsets[e + 1]), beg), cap_rows);
  }
  const int p0 = blockIdx.y * BM, q0 = blockIdx.x * BN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int64_t m0 = beg; m0 < end; m0 += BK) {
    for (int i = tid; i < BK * BM; i += kThreads) {
      const int k = i / BM, p = i % BM;  // consecutive threads along p (contiguous)
      As[k][p] = m0 + k < end && p0 + p < P ? A[(m0 + k) * P + p0 + p] : 0.f;
    }
    for (int i = tid; i < BK * BN; i += kThreads) {
      const int k = i / BN, q = i % BN;
      Bs[k][q] = m0 + k < end && q0 + q < Q ? B[(m0 + k) * Q + q0 + q] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[k][ty * 4 + i];
        b[i] = Bs[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* Ce = C + static_cast<int64_t>(e) * P * Q;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = p0 + ty * 4 + i;
    if (p >= P) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = q0 + tx * 4 + j;
      if (q < Q) Ce[static_cast<int64_t>(p) * Q + q] = acc[i][j];
    }
  }
}

// In place over gu [rows, 2I] (G | U in, dG | dU out); h [rows, I] out.
// s = 1 / (1 + exp(-g)), SiLU(g) = g s, SiLU'(g) = s + SiLU(g) (1 - s).
__global__ __launch_bounds__(kThreads) void swiglu_bwd_f32(int64_t rows, int I,
                                                           const float* __restrict__ dh,
                                                           float* __restrict__ gu,
                                                           float* __restrict__ h) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= rows * I) return;
  const int64_t r = i / I, c = i - r * I;
  float* row = gu + r * 2 * I;
  const float g = row[c], u = row[I + c], d = dh[i];
  const float s = 1.f / (1.f + expf(-g));
  const float silu = g * s;
  row[c] = d * u * (s + silu * (1.f - s));
  row[I + c] = d * silu;
  h[i] = silu * u;
}

int64_t row_tiles(int64_t cap_rows, const int32_t* offsets, int n_experts) {
  return (cap_rows + BM - 1) / BM + (offsets ? n_experts : 0);
}

}  // namespace

hipError_t launch_rows_gemm_f32(int n_experts, int64_t cap_rows, const float* a,
                                const int32_t* offsets, const float* w, int64_t w_es,
                                int64_t w_sk, int64_t w_sn, float* c, int K, int N,
                                hipStream_t s) {
  if (cap_rows == 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(row_tiles(cap_rows, offsets, n_experts)), (N + BN - 1) / BN);
  rows_gemm<<<g, kThreads, 0, s>>>(a, offsets, offsets ? n_experts : 1, cap_rows, w, w_es, w_sk,
                                   w_sn, c, K, N);
  return hipGetLastError();
}

hipError_t launch_contract_gemm_f32(int n_experts, int64_t cap_rows, const float* a, int P,
                                    const float* b, int Q, const int32_t* offsets, float* c,
                                    hipStream_t s) {
  const dim3 g((Q + BN - 1) / BN, (P + BM - 1) / BM, n_experts);
  contract_gemm<<<g, kThreads, 0, s>>>(a, P, b, Q, offsets, cap_rows, c);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd_f32(int64_t rows, int inter, const float* dh, float* gu, float* h,
                                 hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t n = rows * inter;
  swiglu_bwd_f32<<<static_cast<unsigned>((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(
      rows, inter, dh, gu, h);
  return hipGetLastError();
}

}  // namespace moe
