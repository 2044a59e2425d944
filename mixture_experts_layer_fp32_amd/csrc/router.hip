// Router: fp32 logits, softmax and top-k for a tile of tokens per workgroup.
//
// Page "Worked Example: Tracing a Token Through Expert Parallelism", Step 1:
// the gate produces logits for all experts, softmax normalises them and the
// top-k experts are chosen with their weights. Page "Expert Parallel (EP)",
// Configuration: the router computes in fp32.
//
// Each logit is the dot product of a token with one gate-weight row. Both
// factors widen exactly to fp64 (bf16/fp32 x fp32 needs at most 48 bits of
// mantissa), so every product is exact; the sum is accumulated in fp64 on the
// fp64 matrix cores (v_mfma_f64_16x16x4_f64) and rounded once to fp32. The
// fp32 logit the top-k decision is made on is therefore the correctly rounded
// dot product up to fp64 summation error (~1e-16 relative), which keeps the
// choice stable against near ties of the fp32 values.
//
// Work split. A workgroup (4 waves) owns MB blocks of 16 tokens and all E
// experts. The logit matrix of the tile is cut into 16x16 blocks (16 tokens x
// 16 experts). A "unit" is one 16-expert block over one slice of the hidden
// dimension; with few experts (E <= 32) the hidden dimension is split over
// the waves (KS slices, summed in LDS in a fixed order), otherwise each wave
// owns whole expert blocks and accumulates up to four of them at once. The
// hidden dimension is walked in chunks of 32: lane group g (lanes 16g..16g+15)
// feeds elements 8g..8g+7 of the chunk, one per MFMA step, so one 16-byte
// load of a token row (bf16) covers eight steps.
//
// After the logits sit in LDS as fp32 (+ bias), one wave per token selects
// the top-k in registers (each lane holds experts lane, lane+64, ...) with k
// rounds of a cross-lane argmax; ties go to the lower expert id.
//
// Router dtype (page "Expert Parallel (EP)", Configuration: router_dtype
// fp32, bf16 or fp16). With bf16 or fp16 the gate weight is held in that
// dtype and each logit is the dot product rounded once, to nearest even, to
// that dtype (the bias, when present, is added to the rounded value and the
// sum rounded again); softmax and top-k then run on those values in fp32.
// The products stay exact in fp64 (bf16 or fp32 times fp16 needs at most 35
// bits), so the rounding is applied to the fp64 sum directly.
#include <math.h>

#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / 64;  // experts held per lane in top-k
constexpr int kChunk = 32;                         // hidden elements per MFMA group of 8 steps

struct RoutePlan {
  int mb;   // 16-token blocks per workgroup
  int neb;  // 16-expert blocks
  int ks;   // hidden-dimension slices (waves sharing one expert block)
};

__host__ __device__ inline RoutePlan route_plan(int T, int E) {
  RoutePlan p;
  p.neb = (E + 15) / 16;
  p.ks = p.neb >= kWaves ? 1 : (p.neb <= 2 ? kWaves / p.neb : 1);
  // Two token blocks share each gate-weight load when that still leaves a
  // workgroup per CU.
  p.mb = (E > 64 && E <= 512 && (T + 31) / 32 >= 256) ? 2 : 1;
  return p;
}

// LDS: fp32 logits [TM][E], per-token max and sum [TM] each, then (when the
// hidden dimension is split) fp64 partial logits [KS][TM][16 * NEB] at the
// next 16-byte boundary.
__host__ __device__ inline size_t route_part_offset(int tm, int E) {
  return ((static_cast<size_t>(tm) * E + 2 * tm) * sizeof(float) + 15) / 16 * 16;
}
__host__ inline size_t route_lds_bytes(const RoutePlan& p, int E) {
  const int tm = 16 * p.mb;
  size_t b = route_part_offset(tm, E);
  if (p.ks > 1) b += static_cast<size_t>(p.ks) * tm * p.neb * 16 * sizeof(double);
  return b;
}

// Eight consecutive elements of a row, loaded raw and widened to fp64 later,
// so the loads of the next chunk can be in flight during this chunk's MFMAs.
struct Raw8 {
  uint4 a, b;  // bf16 rows use a only
};
__device__ __forceinline__ Raw8 load_raw8(const uint16_t* p) {
  Raw8 r;
  r.a = *reinterpret_cast<const uint4*>(p);
  r.b = r.a;
  return r;
}
__device__ __forceinline__ Raw8 load_raw8(const float* p) {
  Raw8 r;
  r.a = reinterpret_cast<const uint4*>(p)[0];
  r.b = reinterpret_cast<const uint4*>(p)[1];
  return r;
}
__device__ __forceinline__ Raw8 load_raw8(const _Float16* p) {
  Raw8 r;
  r.a = *reinterpret_cast<const uint4*>(p);
  r.b = r.a;
  return r;
}
template <typename T>
__device__ __forceinline__ void widen8(const Raw8& r, double (&v)[8]);
template <>
__device__ __forceinline__ void widen8<_Float16>(const Raw8& r, double (&v)[8]) {
  const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = static_cast<double>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i])));
    v[2 * i + 1] =
        static_cast<double>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
  }
}
template <>
__device__ __forceinline__ void widen8<uint16_t>(const Raw8& r, double (&v)[8]) {
  const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = static_cast<double>(__uint_as_float(w[i] << 16));
    v[2 * i + 1] = static_cast<double>(__uint_as_float(w[i] & 0xffff0000u));
  }
}
template <>
__device__ __forceinline__ void widen8<float>(const Raw8& r, double (&v)[8]) {
  const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = static_cast<double>(__uint_as_float(w[i]));
}

// ---- cross-lane argmax / sum within a group of LPT lanes ------------------
// Steps inside a row of 16 lanes use DPP (xor 1, xor 2, half-row mirror,
// row mirror); xor 16 inside 32 lanes uses ds_swizzle; the two halves of a
// wave are joined through readlane. Every pairing is an involution, so all
// lanes of the group end with the same result.
__device__ __forceinline__ int dpp(int v, int ctrl_sel) {
  switch (ctrl_sel) {
    case 0: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    case 1: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    case 2: return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);  // row_half_mirror
    default: return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true); // row_mirror
  }
}

__device__ __forceinline__ void take_better(float& bv, int& be, float ov, int oe) {
  if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
}

template <int LPT>
__device__ __forceinline__ void group_argmax(float& bv, int& be) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    take_better(bv, be, __int_as_float(dpp(__float_as_int(bv), c)), dpp(be, c));
  if (LPT >= 32)
    take_better(bv, be, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(bv), 0x401F)),
                __builtin_amdgcn_ds_swizzle(be, 0x401F));
  if (LPT == 64) {
    float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
    int e0 = __builtin_amdgcn_readlane(be, 0);
    const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 32));
    const int e1 = __builtin_amdgcn_readlane(be, 32);
    take_better(v0, e0, v1, e1);
    bv = v0;
    be = e0;
  }
}

template <int LPT>
__device__ __forceinline__ float group_sum(float s) {
#pragma unroll
  for (int c = 0; c < 4; ++c) s += __int_as_float(dpp(__float_as_int(s), c));
  if (LPT >= 32) s += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(s), 0x401F));
  if (LPT == 64)
    s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 0)) +
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 32));
  return s;
}

// Top-k and softmax statistics of the n_tok token rows in ls [TM][E]. A group
// of LPT lanes owns one token (64 / LPT tokens per wave at a time); lane sl of
// the group holds experts sl, sl + LPT, ... and k rounds of a group argmax
// pick the choices in order (ties to the lower expert id); lane j of the
// group keeps the j-th choice.
template <int LPT>
__device__ __forceinline__ void topk_rows(const float* ls, int n_tok, int E, int k, int norm_topk,
                                          int64_t t0, int wave, int lane, float* tok_max,
                                          float* tok_sum, int32_t* __restrict__ topk_idx,
                                          float* __restrict__ topk_w) {
  constexpr int kPer = LPT == 64 ? kMaxPerLane : 1;
  const int sub = lane / LPT, sl = lane % LPT;
  const int per_lane = (E + LPT - 1) / LPT;
  for (int tb = wave * (64 / LPT); tb < n_tok; tb += kWaves * (64 / LPT)) {
    const int tk = tb + sub;
    const bool valid = tk < n_tok;
    const float* lrow = ls + (valid ? tk : 0) * E;
    float v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = sl + LPT * i;
      v[i] = (valid && i < per_lane && e < E) ? lrow[e] : -INFINITY;
    }
    uint32_t taken = 0;
    float m = 0.f, s_sel = 0.f, my_v = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = sl + LPT * i;
        if (i < per_lane && e < E && !((taken >> i) & 1u)) take_better(bv, be, v[i], e);
      }
      group_argmax<LPT>(bv, be);
      if (j == 0) m = bv;  // the largest logit
      s_sel += expf(bv - m);
      if (sl == j) { my_v = bv; my_e = be; }
      if (be % LPT == sl) taken |= 1u << (be / LPT);
    }
    // Softmax over all experts shares the same shift m.
    float s_all = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = sl + LPT * i;
      if (i < per_lane && e < E) s_all += expf(v[i] - m);
    }
    s_all = group_sum<LPT>(s_all);
    const float denom = norm_topk ? s_sel : s_all;
    if (valid) {
      const int64_t t = t0 + tk;
      if (sl < k) {
        topk_idx[t * k + sl] = my_e;
        topk_w[t * k + sl] = expf(my_v - m) / denom;
      }
      if (sl == 0) {
        tok_max[tk] = m;
        tok_sum[tk] = s_all;
      }
    }
  }
}

// Logit rounding: RD = 0 fp32, 1 bf16 (8 significant bits, smallest normal
// 2^-126), 2 fp16 (11 bits, smallest normal 2^-14, subnormal step 2^-24,
// largest finite 65504). Round to nearest even of the fp64 value, computed on
// the significand (frexp / rint / ldexp), then converted exactly to fp32.
template <int RD>
__device__ __forceinline__ float round_logit(double v) {
  if (RD == 0) return static_cast<float>(v);
  if (!(v == v) || v == 0.0) return static_cast<float>(v);
  constexpr int P = RD == 1 ? 8 : 11;        // significant bits
  constexpr int EMIN = RD == 1 ? -126 : -14;  // exponent of the smallest normal
  int e;
  const double m = frexp(v, &e);             // v = m 2^e, 0.5 <= |m| < 1
  // quantum 2^(e - P) for normals, 2^(EMIN - P + 1) below the normal range
  const int q = max(e, EMIN + 1) - P;
  const double r = ldexp(rint(ldexp(m, e - q)), q);
  if (RD == 2 && fabs(r) > 65504.0) return r > 0 ? INFINITY : -INFINITY;
  return static_cast<float>(r);
}
template <int RD>
__device__ __forceinline__ float biased_logit(double dot, const float* bias, int e) {
  float l = round_logit<RD>(dot);
  if (bias != nullptr)
    l = RD == 0 ? l + bias[e] : round_logit<RD>(static_cast<double>(l) + static_cast<double>(bias[e]));
  return l;
}

// MB: 16-token blocks per workgroup; NU: 16-expert blocks a wave accumulates
// in one pass (1 when the hidden dimension is split over the waves); NPF:
// chunks whose loads are in flight ahead of the MFMAs.
// WT: gate weight element type (float, bf16 as uint16_t, _Float16); RD: the
// logit rounding (round_logit). Logits are stored as fp32 (RD = 0) or as the
// 16-bit router dtype.
template <typename XT, typename WT, int RD, int MB, int NU, int NPF>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const XT* __restrict__ x, const WT* __restrict__ wr, const float* __restrict__ bias,
    int T, int D, int E, int k, int norm_topk, void* __restrict__ logits,
    float* __restrict__ probs, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const RoutePlan plan = route_plan(T, E);
  const int TM = 16 * MB;
  float* ls = reinterpret_cast<float*>(smem_raw);  // [TM][E] fp32 logits
  float* tok_max = ls + TM * E;                    // [TM]
  float* tok_sum = tok_max + TM;                   // [TM]
  double* part = reinterpret_cast<double*>(smem_raw + route_part_offset(TM, E));

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int t0 = blockIdx.x * TM;
  const int n_tok = min(TM, T - t0);
  const int col = lane & 15, grp = lane >> 4;
  const int n_chunks = D / kChunk;
  const int n_units = plan.neb * plan.ks;
  const int ks = plan.ks;

  // Token rows this lane feeds (clamped to a valid row; results of rows past
  // T are never stored).
  const XT* xrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
    xrow[m] = x + static_cast<int64_t>(min(t0 + 16 * m + col, T - 1)) * D + 8 * grp;

  for (int u0 = wave; u0 < n_units; u0 += kWaves * NU) {
    // Units u0, u0 + 4, ... (at most NU) share this pass's loads of x.
    const int slice = u0 % ks;
    const WT* wrow[NU];
    bool on[NU];
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int u = u0 + j * kWaves;
      on[j] = u < n_units;
      wrow[j] = wr + static_cast<int64_t>(min((u / ks) * 16 + col, E - 1)) * D + 8 * grp;
    }
    // NACC independent accumulators per output block (summed at the end) so
    // that consecutive MFMAs do not wait on each other's results.
    constexpr int NACC = MB * NU >= 4 ? 1 : 4 / (MB * NU);
    f64x4 acc[NACC][MB][NU];
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < NU; ++j) acc[a][m][j] = f64x4{0.0, 0.0, 0.0, 0.0};

    // Chunks slice, slice + ks, ...; ring of NPF chunks of raw loads. Every
    // fetch is issued (chunks past the end reload the last chunk, unused), so
    // the count of loads in flight is the same on every path and the waits
    // before each chunk only cover that chunk's loads.
    Raw8 xr[NPF][MB], wraw[NPF][NU];
    auto fetch = [&](int p, int c) {
      const int d0 = min(c, n_chunks - 1) * kChunk;
#pragma unroll
      for (int m = 0; m < MB; ++m) xr[p][m] = load_raw8(xrow[m] + d0);
#pragma unroll
      for (int j = 0; j < NU; ++j) wraw[p][j] = load_raw8(wrow[j] + d0);
    };
#pragma unroll
    for (int p = 0; p < NPF; ++p) fetch(p, slice + p * ks);
    // ALL: every unit of this pass is valid, so the MFMAs run without a test
    // (a test per MFMA, left to the compiler, stayed inside the loop as a
    // branch around each MFMA, with accumulator copies at every join).
    auto compute = [&](auto all_c, int p, int c) {
      constexpr bool ALL = decltype(all_c)::value;
      double xa[MB][8], wb[NU][8];
#pragma unroll
      for (int m = 0; m < MB; ++m) widen8<XT>(xr[p][m], xa[m]);
#pragma unroll
      for (int j = 0; j < NU; ++j) widen8<WT>(wraw[p][j], wb[j]);
      fetch(p, c + NPF * ks);
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int j = 0; j < NU; ++j) {
          if (!ALL && !on[j]) continue;
#pragma unroll
          for (int m = 0; m < MB; ++m)
            acc[s % NACC][m][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                xa[m][s], wb[j][s], acc[s % NACC][m][j], 0, 0, 0);
        }
    };
    // This wave's chunks are slice + i * ks for i < nc: whole rounds of NPF
    // first (no branches between the loads and their uses), then the rest.
    const int nc = (n_chunks - slice + ks - 1) / ks;
    auto chunks = [&](auto all_c) {
      int i = 0;
      for (; i + NPF <= nc; i += NPF) {
#pragma unroll
        for (int p = 0; p < NPF; ++p) compute(all_c, p, slice + (i + p) * ks);
      }
#pragma unroll
      for (int p = 0; p < NPF - 1; ++p)
        if (i + p < nc) compute(all_c, p, slice + (i + p) * ks);
    };
    bool all_on = true;
#pragma unroll
    for (int j = 0; j < NU; ++j) all_on = all_on && on[j];
    if (all_on)  // (uniform: the units depend on the wave only)
      chunks(std::true_type{});
    else
      chunks(std::false_type{});

    // Output block layout of the f64 16x16x4 MFMA: item r of a lane holds row
    // grp + 4 * r (token), column col (expert).
#pragma unroll
    for (int a = 1; a < NACC; ++a)
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < NU; ++j) acc[0][m][j] += acc[a][m][j];
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      if (!on[j]) continue;
      const int e = ((u0 + j * kWaves) / ks) * 16 + col;
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tk = 16 * m + grp + 4 * r;
          if (ks > 1) {
            part[(static_cast<int64_t>(slice) * TM + tk) * (plan.neb * 16) + e] = acc[0][m][j][r];
          } else if (e < E) {
            float l = biased_logit<RD>(acc[0][m][j][r], bias, e);
            if (l != l) l = -INFINITY;  // a NaN logit is never preferred
            ls[tk * E + e] = l;
          }
        }
    }
  }
  if (ks > 1) {
    __syncthreads();
    const int ew = plan.neb * 16;
    for (int o = tid; o < TM * E; o += kThreads) {
      const int tk = o / E, e = o - tk * E;
      double s = 0.0;
      for (int q = 0; q < ks; ++q) s += part[(static_cast<int64_t>(q) * TM + tk) * ew + e];
      float l = biased_logit<RD>(s, bias, e);
      if (l != l) l = -INFINITY;
      ls[o] = l;
    }
  }
  __syncthreads();

  if (E <= 16)
    topk_rows<16>(ls, n_tok, E, k, norm_topk, t0, wave, lane, tok_max, tok_sum, topk_idx, topk_w);
  else if (E <= 32)
    topk_rows<32>(ls, n_tok, E, k, norm_topk, t0, wave, lane, tok_max, tok_sum, topk_idx, topk_w);
  else
    topk_rows<64>(ls, n_tok, E, k, norm_topk, t0, wave, lane, tok_max, tok_sum, topk_idx, topk_w);

  if (logits != nullptr || probs != nullptr) {
    __syncthreads();
    for (int o = tid; o < n_tok * E; o += kThreads) {
      const int tk = o / E;
      const int64_t g = static_cast<int64_t>(t0) * E + o;
      if (logits != nullptr) {
        if (RD == 0)
          static_cast<float*>(logits)[g] = ls[o];
        else if (RD == 1)  // exact: the value has at most 8 significant bits
          static_cast<uint16_t*>(logits)[g] = static_cast<uint16_t>(__float_as_uint(ls[o]) >> 16);
        else
          static_cast<_Float16*>(logits)[g] = static_cast<_Float16>(ls[o]);
      }
      if (probs != nullptr) probs[g] = expf(ls[o] - tok_max[tk]) / tok_sum[tk];
    }
  }
}

template <typename XT, typename WT, int RD>
void launch_route_t(const moe_desc& d, const XT* x, const WT* w_router, const float* bias,
                    void* logits, float* probs, int32_t* topk_idx, float* topk_w,
                    hipStream_t s) {
  const RoutePlan p = route_plan(d.T, d.E);
  const int tm = 16 * p.mb;
  const int grid = (d.T + tm - 1) / tm;
  const size_t lds = route_lds_bytes(p, d.E);
#define MOE_ROUTE_ARGS \
  x, w_router, bias, d.T, d.D, d.E, d.top_k, d.norm_topk, logits, probs, topk_idx, topk_w
  if (p.ks > 1)
    route_kernel<XT, WT, RD, 1, 1, 4><<<grid, kThreads, lds, s>>>(MOE_ROUTE_ARGS);
  else if (p.mb == 1)
    route_kernel<XT, WT, RD, 1, 4, 2><<<grid, kThreads, lds, s>>>(MOE_ROUTE_ARGS);
  else if (p.neb <= 8)  // 8 expert blocks: 2 per wave (4 per wave left half the slots idle,
                        // their loads still issued; skewed 128-expert router 237 -> 229 us)
    route_kernel<XT, WT, RD, 2, 2, 2><<<grid, kThreads, lds, s>>>(MOE_ROUTE_ARGS);
  else
    route_kernel<XT, WT, RD, 2, 4, 2><<<grid, kThreads, lds, s>>>(MOE_ROUTE_ARGS);
#undef MOE_ROUTE_ARGS
}

}  // namespace

hipError_t launch_route(const moe_desc& d, const void* x, const float* w_router,
                        const float* bias, float* logits, float* probs, int32_t* topk_idx,
                        float* topk_w, hipStream_t s) {
  return launch_route_typed(d, MOE_F32, x, w_router, bias, logits, probs, topk_idx, topk_w, s);
}

hipError_t launch_route_typed(const moe_desc& d, int router_dtype, const void* x,
                              const void* w_router, const float* bias, void* logits, float* probs,
                              int32_t* topk_idx, float* topk_w, hipStream_t s) {
  auto go = [&](auto xp) {
    using XT = std::remove_const_t<std::remove_pointer_t<decltype(xp)>>;
    if (router_dtype == MOE_BF16)
      launch_route_t<XT, uint16_t, 1>(d, xp, static_cast<const uint16_t*>(w_router), bias, logits,
                                      probs, topk_idx, topk_w, s);
    else if (router_dtype == MOE_F16)
      launch_route_t<XT, _Float16, 2>(d, xp, static_cast<const _Float16*>(w_router), bias, logits,
                                      probs, topk_idx, topk_w, s);
    else
      launch_route_t<XT, float, 0>(d, xp, static_cast<const float*>(w_router), bias, logits,
                                   probs, topk_idx, topk_w, s);
  };
  if (d.act_dtype == MOE_BF16)
    go(static_cast<const uint16_t*>(x));
  else
    go(static_cast<const float*>(x));
  return hipGetLastError();
}

}  // namespace moe
