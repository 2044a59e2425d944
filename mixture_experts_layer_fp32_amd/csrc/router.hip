// Router: fp32 logits, softmax and top-k for a tile of tokens per workgroup.
//
// Page "Worked Example: Tracing a Token Through Expert Parallelism", Step 1:
// the gate produces logits for all experts, softmax normalises them and the
// top-k experts are chosen with their weights. Page "Expert Parallel (EP)",
// Configuration: the router computes in fp32.
//
// Each logit is the dot product of a token with one gate-weight row. Both
// factors widen exactly to fp64 (bf16/fp32 x fp32 needs at most 48 bits), so
// the products are exact and the sum is accumulated in fp64, then rounded
// once to fp32. The fp32 logit the top-k decision is made on is therefore the
// correctly rounded dot product (up to fp64 summation error, ~1e-16 relative),
// which keeps the choice stable against near ties of the fp32 values.
//
// Layout per workgroup (256 threads): TT tokens x E experts of logits, at
// most 4 per thread. Token rows and gate rows are staged through LDS in
// chunks of DC hidden elements; then one wavefront per token selects the
// top-k in registers (each lane holds experts lane, lane+64, ...) with k
// rounds of a cross-lane argmax.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxOut = 4;                       // logits per thread
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / 64;  // experts held per lane in top-k

struct RouteShape {
  int TT;  // tokens per workgroup
  int DC;  // hidden elements staged per chunk
};

__host__ __device__ inline RouteShape route_shape(int E) {
  RouteShape s;
  s.TT = E >= kThreads ? 1 : (kThreads / E < 64 ? kThreads / E : 64);
  // Gate-weight chunk E x (DC + 4) floats stays under 50 KB of LDS.
  s.DC = E <= 128 ? 64 : (E <= 256 ? 32 : (E <= 512 ? 16 : 8));
  return s;
}

__host__ inline size_t route_lds_bytes(int E) {
  RouteShape s = route_shape(E);
  size_t xs = static_cast<size_t>(s.TT) * s.DC;
  size_t ws = static_cast<size_t>(E) * (s.DC + 4);
  size_t ls = static_cast<size_t>(s.TT) * E;
  return (xs + ws + ls + 2 * s.TT) * sizeof(float);
}

template <typename XT>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const XT* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    int T, int D, int E, int k, int norm_topk, float* __restrict__ logits,
    float* __restrict__ probs, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  extern __shared__ float smem[];
  const RouteShape shp = route_shape(E);
  const int TT = shp.TT, DC = shp.DC, WS = DC + 4;
  float* xs = smem;                        // [TT][DC]
  float* ws = xs + TT * DC;                // [E][DC + 4]
  float* ls = ws + E * WS;                 // [TT][E] fp32 logits
  float* tok_max = ls + TT * E;            // [TT]
  float* tok_sum = tok_max + TT;           // [TT]

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TT;
  const int n_tok = min(TT, T - t0);
  const int n_out = TT * E;

  double acc[kMaxOut];
#pragma unroll
  for (int i = 0; i < kMaxOut; ++i) acc[i] = 0.0;

  for (int d0 = 0; d0 < D; d0 += DC) {
    __syncthreads();
    for (int i = tid; i < TT * DC; i += kThreads) {
      const int tk = i / DC, dd = i - tk * DC;
      xs[i] = tk < n_tok ? load_act(x + static_cast<int64_t>(t0 + tk) * D + d0 + dd) : 0.f;
    }
    for (int i = tid; i < E * DC; i += kThreads) {
      const int e = i / DC, dd = i - e * DC;
      ws[e * WS + dd] = wr[static_cast<int64_t>(e) * D + d0 + dd];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxOut; ++i) {
      const int o = tid + i * kThreads;
      if (o < n_out) {
        const int tk = o / E, e = o - tk * E;
        const float4* xv = reinterpret_cast<const float4*>(xs + tk * DC);
        const float4* wv = reinterpret_cast<const float4*>(ws + e * WS);
        double a = acc[i];
        for (int q = 0; q < DC / 4; ++q) {
          const float4 xa = xv[q], wa = wv[q];
          a = fma(static_cast<double>(xa.x), static_cast<double>(wa.x), a);
          a = fma(static_cast<double>(xa.y), static_cast<double>(wa.y), a);
          a = fma(static_cast<double>(xa.z), static_cast<double>(wa.z), a);
          a = fma(static_cast<double>(xa.w), static_cast<double>(wa.w), a);
        }
        acc[i] = a;
      }
    }
  }

  // fp32 logits (+ bias in fp32) into LDS.
#pragma unroll
  for (int i = 0; i < kMaxOut; ++i) {
    const int o = tid + i * kThreads;
    if (o < n_out) {
      const int e = o % E;
      float l = static_cast<float>(acc[i]);
      if (bias != nullptr) l = l + bias[e];
      if (l != l) l = -INFINITY;  // a NaN logit is never preferred
      ls[o] = l;
    }
  }
  __syncthreads();

  // Top-k: one wavefront per token.
  const int wave = tid >> 6, lane = tid & 63;
  const int per_lane = (E + 63) / 64;
  for (int tk = wave; tk < n_tok; tk += kThreads / 64) {
    const float* lrow = ls + tk * E;
    float v[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      v[i] = (i < per_lane && e < E) ? lrow[e] : -INFINITY;
    }
    // k rounds of a cross-lane argmax; lane j keeps the j-th choice.
    uint32_t taken = 0;
    float m = 0.f, s_sel = 0.f, my_v = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        if (i < per_lane && e < E && !((taken >> i) & 1u)) {
          if (v[i] > bv || (v[i] == bv && e < be)) { bv = v[i]; be = e; }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oe = __shfl_xor(be, off, 64);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if (j == 0) m = bv;  // the largest logit
      s_sel += expf(bv - m);
      if (lane == j) { my_v = bv; my_e = be; }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
    }
    // Softmax over all experts shares the same shift m.
    float s_all = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (i < per_lane && e < E) s_all += expf(v[i] - m);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s_all += __shfl_xor(s_all, off, 64);
    const float denom = norm_topk ? s_sel : s_all;
    const int64_t t = t0 + tk;
    if (lane < k) {
      topk_idx[t * k + lane] = my_e;
      topk_w[t * k + lane] = expf(my_v - m) / denom;
    }
    if (lane == 0) {
      tok_max[tk] = m;
      tok_sum[tk] = s_all;
    }
  }

  if (logits != nullptr || probs != nullptr) {
    __syncthreads();
    for (int o = tid; o < n_tok * E; o += kThreads) {
      const int tk = o / E;
      const int64_t g = static_cast<int64_t>(t0) * E + o;
      if (logits != nullptr) logits[g] = ls[o];
      if (probs != nullptr) probs[g] = expf(ls[o] - tok_max[tk]) / tok_sum[tk];
    }
  }
}

}  // namespace

hipError_t launch_route(const moe_desc& d, const void* x, const float* w_router,
                        const float* bias, float* logits, float* probs, int32_t* topk_idx,
                        float* topk_w, hipStream_t s) {
  const RouteShape shp = route_shape(d.E);
  const int grid = (d.T + shp.TT - 1) / shp.TT;
  const size_t lds = route_lds_bytes(d.E);
  if (d.act_dtype == MOE_BF16) {
    route_kernel<uint16_t><<<grid, kThreads, lds, s>>>(
        static_cast<const uint16_t*>(x), w_router, bias, d.T, d.D, d.E, d.top_k, d.norm_topk,
        logits, probs, topk_idx, topk_w);
  } else {
    route_kernel<float><<<grid, kThreads, lds, s>>>(
        static_cast<const float*>(x), w_router, bias, d.T, d.D, d.E, d.top_k, d.norm_topk,
        logits, probs, topk_idx, topk_w);
  }
  return hipGetLastError();
}

}  // namespace moe
