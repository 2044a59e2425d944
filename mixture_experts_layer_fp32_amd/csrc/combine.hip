// Unpermute and combine: out[t] = residual[t] + shared[t]
//                                 + sum_j w[t,j] * y_perm[pos[t,j]]   (pos >= 0)
//
// Page "Expert Parallel (EP)", Communication Pattern stage 4 (unpermute and
// apply routing weights); page "Worked Example", Step 4 (the weighted sum of
// the chosen experts' outputs) and Step 5 (the residual connection).
//
// One wavefront per token gathers the token's expert rows (fp32, or fp16 when
// the layer keeps its expert outputs in fp16), accumulates in fp32 (residual,
// shared expert, then the slots in order) and rounds once to the output
// dtype. Each output element is written by exactly one lane, so no atomics
// and the same result every run.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Eight expert-output values of one row: fp32 (two 16-byte loads) or fp16
// (one), widened exactly to fp32.
__device__ __forceinline__ void load8(const float* p, float (&f)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void load8(const _Float16* p, float (&f)[8]) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8 v = __builtin_nontemporal_load(reinterpret_cast<const h8*>(p));
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(v[i]);
}

// bf16 layer: a lane handles 8 elements; expert outputs and the shared
// expert's output are YT (fp32 or fp16), residual and output bf16. Each
// expert row and each output row is touched once, so the fp16 gathers and
// the output stores are non-temporal (measured: Mixtral-style 68.6 ->
// 65.4 us, skewed 128-expert layer 151.9 -> 143.1 us; unrolling four or
// eight chunks instead of two helped the first and slowed the second).
template <typename YT>
__global__ __launch_bounds__(kThreads) void combine_bf16_kernel(
    const YT* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ w,
    const uint4* __restrict__ res, const YT* __restrict__ sh, int res_begin, int res_rows,
    uint4* __restrict__ out, int T, int k, int row_vec) {
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  int p[MOE_MAX_TOPK];
  float wt[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    p[j] = j < k ? pos[static_cast<int64_t>(t) * k + j] : -1;
    wt[j] = j < k ? w[static_cast<int64_t>(t) * k + j] : 0.f;
  }
  const int rr = t - res_begin;
  const bool has_res = rr >= 0 && rr < res_rows;
  // Two chunks per loop pass keep both chunks' gathers in flight together
  // (measured: Mixtral-style 97 -> 89 us; four chunks were slower).
#pragma unroll 2
  for (int c = lane; c < row_vec; c += 64) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    if (has_res && res != nullptr) {
      float f[8];
      unpack8(res[static_cast<int64_t>(rr) * row_vec + c], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
    if (has_res && sh != nullptr) {
      float f[8];
      load8(sh + (static_cast<int64_t>(rr) * row_vec + c) * 8, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (p[j] >= 0) {
        float f[8];
        load8(y + (static_cast<int64_t>(p[j]) * row_vec + c) * 8, f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wt[j], f[i], acc[i]);
      }
    }
    uint4 o;
    o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w},
                                reinterpret_cast<u32x4*>(out + static_cast<int64_t>(t) * row_vec + c));
  }
}

// fp32: a vector is 4 elements.
__global__ __launch_bounds__(kThreads) void combine_f32_kernel(
    const float4* __restrict__ y, const int32_t* __restrict__ pos, const float* __restrict__ w,
    const float4* __restrict__ res, const float4* __restrict__ sh, int res_begin, int res_rows,
    float4* __restrict__ out, int T, int k, int row_vec) {
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  int p[MOE_MAX_TOPK];
  float wt[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    p[j] = j < k ? pos[static_cast<int64_t>(t) * k + j] : -1;
    wt[j] = j < k ? w[static_cast<int64_t>(t) * k + j] : 0.f;
  }
  const int rr = t - res_begin;
  const bool has_res = rr >= 0 && rr < res_rows;
  for (int c = lane; c < row_vec; c += 64) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (has_res && res != nullptr) {
      const float4 v = res[static_cast<int64_t>(rr) * row_vec + c];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (has_res && sh != nullptr) {
      const float4 v = sh[static_cast<int64_t>(rr) * row_vec + c];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (p[j] >= 0) {
        const float4 v = y[static_cast<int64_t>(p[j]) * row_vec + c];
        acc.x = fmaf(wt[j], v.x, acc.x);
        acc.y = fmaf(wt[j], v.y, acc.y);
        acc.z = fmaf(wt[j], v.z, acc.z);
        acc.w = fmaf(wt[j], v.w, acc.w);
      }
    }
    out[static_cast<int64_t>(t) * row_vec + c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const moe_desc& d, const void* y_perm, const int32_t* pos,
                          const float* topk_w, const void* residual, const void* shared_out,
                          int res_begin, int res_rows, void* out, hipStream_t s) {
  const int grid = (d.T + 3) / 4;
  if (d.act_dtype == MOE_BF16 && d.expert_out_dtype == MOE_F16) {
    combine_bf16_kernel<_Float16><<<grid, kThreads, 0, s>>>(
        static_cast<const _Float16*>(y_perm), pos, topk_w, static_cast<const uint4*>(residual),
        static_cast<const _Float16*>(shared_out), res_begin, res_rows, static_cast<uint4*>(out),
        d.T, d.top_k, d.D / 8);
  } else if (d.act_dtype == MOE_BF16) {
    combine_bf16_kernel<float><<<grid, kThreads, 0, s>>>(
        static_cast<const float*>(y_perm), pos, topk_w, static_cast<const uint4*>(residual),
        static_cast<const float*>(shared_out), res_begin, res_rows, static_cast<uint4*>(out),
        d.T, d.top_k, d.D / 8);
  } else {
    combine_f32_kernel<<<grid, kThreads, 0, s>>>(
        static_cast<const float4*>(y_perm), pos, topk_w, static_cast<const float4*>(residual),
        static_cast<const float4*>(shared_out), res_begin, res_rows, static_cast<float4*>(out),
        d.T, d.top_k, d.D / 4);
  }
  return hipGetLastError();
}

}  // namespace moe
