// Memory-bound kernels of the MoE layer's backward pass (gfx950): the adjoints
// of the combine, of the routing weights and of the router GEMM, and the
// assembly of the input gradient.
//
// Forward (page "Worked Example", Steps 1, 4 and 5; page "Expert Parallel
// (EP)", Communication Pattern stage 4): out[t] = x[t] + S(x[t])
// + sum_j w[t,j] y_perm[pos[t,j]], with w[t,:] the softmax over the chosen
// experts' logits (renormalised top-k weights), logits = x W_r^T.
// Backward, per token t and slot j (p = pos[t,j]):
//   dw[t,j]      = dout[t] . y_perm[p]                  (combine_bwd_kernel)
//   dy_perm[p]   = w[t,j] dout[t]  (bf16, the expert GEMMs' operand)
//   dl[t,j]      = w[t,j] (dw[t,j] - sum_i w[t,i] dw[t,i])   (gradient of the
//                  logit of expert topk_idx[t,j]; the others get none)
//   dW_r[e]      = sum over the rows p of expert e of dl_perm[p] x_perm[p]
//                  (router_bwd_partial_kernel + router_bwd_reduce_kernel,
//                  deterministic: fixed-order sums, no atomics)
//   dx[t]        = ((dS[t] + sum_j dx_perm[p]) + sum_j dl[t,j] W_r[e_j]) + dout[t]
//                  (input_bwd_kernel; the order (shared + routed) + router
//                  of torchtitan issue 5554, then the residual)
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 4;  // tokens per 256-thread workgroup (one wave each)

// Eight / four consecutive activations (bf16 as raw 16-bit words, or fp32) to
// fp32 and back (bf16: round to nearest even).
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(ws[i] << 16);
    v[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_bf16(v[2 * i]) | (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(o[0], o[1], o[2], o[3]);
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void store4(uint16_t* p, float4 a) {
  *reinterpret_cast<uint2*>(p) =
      make_uint2(f32_to_bf16(a.x) | (static_cast<uint32_t>(f32_to_bf16(a.y)) << 16),
                 f32_to_bf16(a.z) | (static_cast<uint32_t>(f32_to_bf16(a.w)) << 16));
}
__device__ __forceinline__ void store4(float* p, float4 a) { *reinterpret_cast<float4*>(p) = a; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One wave per token. Lane l covers columns 8 l + 512 i; D is a multiple of
// 8. XT: activation type (dout, dy_perm). KMAX >= top_k bounds the per-slot
// register arrays (indexed only with unrolled constants).
template <typename XT, int KMAX>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    int T, int D, int k, const XT* __restrict__ dout, const float* __restrict__ y_perm,
    const int32_t* __restrict__ pos, const float* __restrict__ topk_w,
    XT* __restrict__ dy_perm, float* __restrict__ dtopk_w, float* __restrict__ dlogit,
    float* __restrict__ dl_perm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const XT* g = dout + static_cast<int64_t>(t) * D;
  float dw[KMAX], wt[KMAX];
  int pj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    dw[j] = 0.f;
    wt[j] = 0.f;
    pj[j] = -1;
    if (j < k) {
      pj[j] = pos[static_cast<int64_t>(t) * k + j];
      wt[j] = topk_w[static_cast<int64_t>(t) * k + j];
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) break;
    const int p = pj[j];
    if (p < 0) continue;
    const float* y = y_perm + static_cast<int64_t>(p) * D;
    XT* dy = dy_perm + static_cast<int64_t>(p) * D;
    float acc = 0.f;
    for (int c = 8 * lane; c < D; c += 512) {
      float gv[8], yv[8], o[8];
      load8(g + c, gv);
      load8(y + c, yv);
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        acc += gv[i] * yv[i] + gv[i + 1] * yv[i + 1];
        o[i] = wt[j] * gv[i];
        o[i + 1] = wt[j] * gv[i + 1];
      }
      store8(dy + c, o);
    }
    dw[j] = wave_sum(acc);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (j < k) s += wt[j] * dw[j];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) break;
    if (lane == j) {
      const float dl = wt[j] * (dw[j] - s);
      if (dtopk_w) dtopk_w[static_cast<int64_t>(t) * k + j] = dw[j];
      dlogit[static_cast<int64_t>(t) * k + j] = dl;
      if (dl_perm && pj[j] >= 0) dl_perm[pj[j]] = dl;
    }
  }
}

// One wave per token; lane l covers columns 4 l + 256 i. Sums in the order
// ((shared + routed) + router) + residual, rounds once to bf16.
template <typename XT, int KMAX>
__global__ __launch_bounds__(256) void input_bwd_kernel(
    int T, int D, int k, const float* __restrict__ dx_perm, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dlogit,
    const float* __restrict__ w_router, const float* __restrict__ dx_shared,
    const XT* __restrict__ dout, XT* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  int pj[KMAX], ej[KMAX];
  float lj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    pj[j] = -1;
    ej[j] = 0;
    lj[j] = 0.f;
    if (j < k) {
      pj[j] = pos[static_cast<int64_t>(t) * k + j];
      ej[j] = topk_idx[static_cast<int64_t>(t) * k + j];
      lj[j] = dlogit ? dlogit[static_cast<int64_t>(t) * k + j] : 0.f;
    }
  }
  for (int c = 4 * lane; c < D; c += 256) {
    float4 a = dx_shared ? *reinterpret_cast<const float4*>(dx_shared + static_cast<int64_t>(t) * D + c)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) break;
      if (pj[j] < 0) continue;
      const float4 v = *reinterpret_cast<const float4*>(dx_perm + static_cast<int64_t>(pj[j]) * D + c);
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    if (dlogit) {
      float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j >= k) break;
        const float4 wv = *reinterpret_cast<const float4*>(w_router + static_cast<int64_t>(ej[j]) * D + c);
        r.x += lj[j] * wv.x;
        r.y += lj[j] * wv.y;
        r.z += lj[j] * wv.z;
        r.w += lj[j] * wv.w;
      }
      a.x += r.x;
      a.y += r.y;
      a.z += r.z;
      a.w += r.w;
    }
    if (dout) {
      const float4 gv = load4(dout + static_cast<int64_t>(t) * D + c);
      a.x += gv.x;
      a.y += gv.y;
      a.z += gv.z;
      a.w += gv.w;
    }
    store4(dx + static_cast<int64_t>(t) * D + c, a);
  }
}

constexpr int kRouterChunk = 32;  // permuted rows per partial sum

// Wave (chunk c, 512-column block): sums dl_perm[p] x_perm[p] over the rows p
// of chunk c, one partial per expert met, stored at partial[c + e] (unique:
// the experts of later chunks are never lower). Lane l covers 8 columns.
template <typename XT>
__global__ __launch_bounds__(256) void router_bwd_partial_kernel(
    int n_chunks, int cap, int D, int E, const XT* __restrict__ x_perm,
    const int32_t* __restrict__ offsets, const float* __restrict__ dl_perm,
    float* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int col = blockIdx.y * 512 + 8 * lane;
  if (c >= n_chunks) return;
  const int M = min(offsets[E], cap);  // rows never extend past the buffers
  int p = c * kRouterChunk;
  const int p_end = min(p + kRouterChunk, M);
  if (p >= p_end) return;
  // expert of row p: the last e with offsets[e] <= p (binary search)
  int lo = 0, hi = E;  // offsets[lo] <= p < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid;
  }
  int e = lo;
  while (p < p_end) {
    while (offsets[e + 1] <= p) ++e;
    const int run_end = min(p_end, offsets[e + 1]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // Rows in groups of 4 (their loads issued together), in row order.
    for (; p < run_end; p += 4) {
      const int nr = min(4, run_end - p);
      if (col >= D) continue;
      float xv[4][8];
      float l[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = r < nr ? p + r : p;
        l[r] = r < nr ? dl_perm[q] : 0.f;
        load8(x_perm + static_cast<int64_t>(q) * D + col, xv[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += l[r] * xv[r][i];
    }
    p = run_end;
    if (col < D) {
      float* o = partial + static_cast<int64_t>(c + e) * D + col;
      *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// dW_r[e, d] = sum of the partials of the chunks holding expert e's rows, in
// chunk order; 0 for an expert without rows.
__global__ __launch_bounds__(256) void router_bwd_reduce_kernel(
    int cap, int D, const int32_t* __restrict__ offsets, const float* __restrict__ partial,
    float* __restrict__ dw_router) {
  const int e = blockIdx.x;
  const int col = blockIdx.y * 256 + threadIdx.x;
  if (col >= D) return;
  const int beg = min(max(offsets[e], 0), cap), end = min(max(offsets[e + 1], beg), cap);
  float s = 0.f;
  if (end > beg) {
    const int c0 = beg / kRouterChunk, c1 = (end - 1) / kRouterChunk;
    for (int c = c0; c <= c1; ++c) s += partial[static_cast<int64_t>(c + e) * D + col];
  }
  dw_router[static_cast<int64_t>(e) * D + col] = s;
}

}  // namespace

hipError_t launch_combine_bwd(bool bf16, int T, int D, int k, const void* dout,
                              const float* y_perm, const int32_t* pos, const float* topk_w,
                              void* dy_perm, float* dtopk_w, float* dlogit, float* dl_perm,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  const unsigned g = (T + kWaves - 1) / kWaves;
  auto go = [&](auto kmax) {
    if (bf16)
      combine_bwd_kernel<uint16_t, decltype(kmax)::value><<<g, 64 * kWaves, 0, s>>>(
          T, D, k, static_cast<const uint16_t*>(dout), y_perm, pos, topk_w,
          static_cast<uint16_t*>(dy_perm), dtopk_w, dlogit, dl_perm);
    else
      combine_bwd_kernel<float, decltype(kmax)::value><<<g, 64 * kWaves, 0, s>>>(
          T, D, k, static_cast<const float*>(dout), y_perm, pos, topk_w,
          static_cast<float*>(dy_perm), dtopk_w, dlogit, dl_perm);
  };
  if (k <= 2) go(std::integral_constant<int, 2>{});
  else if (k <= 4) go(std::integral_constant<int, 4>{});
  else if (k <= 8) go(std::integral_constant<int, 8>{});
  else go(std::integral_constant<int, MOE_MAX_TOPK>{});
  return hipGetLastError();
}

hipError_t launch_input_bwd(bool bf16, int T, int D, int k, const float* dx_perm,
                            const int32_t* pos, const int32_t* topk_idx, const float* dlogit,
                            const float* w_router, const float* dx_shared, const void* dout,
                            void* dx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const unsigned g = (T + kWaves - 1) / kWaves;
  auto go = [&](auto kmax) {
    if (bf16)
      input_bwd_kernel<uint16_t, decltype(kmax)::value><<<g, 64 * kWaves, 0, s>>>(
          T, D, k, dx_perm, pos, topk_idx, dlogit, w_router, dx_shared,
          static_cast<const uint16_t*>(dout), static_cast<uint16_t*>(dx));
    else
      input_bwd_kernel<float, decltype(kmax)::value><<<g, 64 * kWaves, 0, s>>>(
          T, D, k, dx_perm, pos, topk_idx, dlogit, w_router, dx_shared,
          static_cast<const float*>(dout), static_cast<float*>(dx));
  };
  if (k <= 2) go(std::integral_constant<int, 2>{});
  else if (k <= 4) go(std::integral_constant<int, 4>{});
  else if (k <= 8) go(std::integral_constant<int, 8>{});
  else go(std::integral_constant<int, MOE_MAX_TOPK>{});
  return hipGetLastError();
}

size_t router_bwd_partial_floats(int64_t cap_rows, int E, int D) {
  return static_cast<size_t>((cap_rows + kRouterChunk - 1) / kRouterChunk + E) *
         static_cast<size_t>(D);
}

hipError_t launch_router_bwd(bool bf16, int64_t cap_rows, int D, int E, const void* x_perm,
                             const int32_t* offsets, const float* dl_perm, float* partial,
                             float* dw_router, hipStream_t s) {
  const int n_chunks = static_cast<int>((cap_rows + kRouterChunk - 1) / kRouterChunk);
  if (n_chunks > 0) {
    const dim3 g((n_chunks + kWaves - 1) / kWaves, (D + 511) / 512);
    if (bf16)
      router_bwd_partial_kernel<uint16_t><<<g, 64 * kWaves, 0, s>>>(
          n_chunks, static_cast<int>(cap_rows), D, E, static_cast<const uint16_t*>(x_perm),
          offsets, dl_perm, partial);
    else
      router_bwd_partial_kernel<float><<<g, 64 * kWaves, 0, s>>>(
          n_chunks, static_cast<int>(cap_rows), D, E, static_cast<const float*>(x_perm), offsets,
          dl_perm, partial);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  router_bwd_reduce_kernel<<<dim3(E, (D + 255) / 256), 256, 0, s>>>(
      static_cast<int>(cap_rows), D, offsets, partial, dw_router);
  return hipGetLastError();
}

}  // namespace moe
