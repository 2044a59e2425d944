// Router: fp32 logits, softmax and top-k for a tile of tokens per workgroup.
//
// Page "Worked Example: Tracing a Token Through Expert Parallelism", Step 1:
// the gate produces logits for all experts, softmax normalises them and the
// top-k experts are chosen with their weights. Page "Expert Parallel (EP)",
// Configuration: the router computes in fp32.
//
// Two paths with the same choices: route_kernel below (fp64 matrix cores;
// fp32 activations, at most 16 experts, and the bf16 / fp16 router dtypes),
// and, further down, the certified router for bf16 activations with more
// than 16 experts (bf16 matrix cores, a proven top-k, exact recompute of the
// undecided candidates).
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


// ===========================================================================
// bf16 activations with the fp32 gate weight: approximate logits on the bf16
// matrix cores, a certified top-k, and an exact fp64 recompute of the
// candidate experts of every token the approximation cannot decide.
//
// Split. Each fp32 weight w is the exact sum of three bf16 numbers:
// hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid (the two differences
// are exact in fp32 and lo needs at most 8 significant bits; only weights
// below 2^-110 in magnitude lose bits, counted in the bound below). A bf16
// activation times a bf16 part is exact in fp32, so x . w is the sum of three
// bf16 GEMMs. They run on v_mfma_f32_16x16x32_bf16 (tokens x experts blocks of
// 16 x 16), hi into one fp32 accumulator and mid + lo into another, each
// started from zero at every 64-wide step of the hidden dimension and added
// to an fp64 accumulator after it, so no fp32 sum spans more than 128
// products. Partial logits (one per slice of the hidden dimension when the
// grid is split along it) are stored as fp32 with the squared norms of the
// token rows and weight rows.
//
// Bound. Whatever order and width the matrix core sums in, a sum of n exact
// products that is rounded to fp32 at most n times (relative error 2^-23 per
// rounding, truncation included) is within gamma_n = n 2^-23 / (1 - n 2^-23)
// times the sum of the products' magnitudes of the exact sum. Summed over the
// steps, with |hi| <= (1 + 2^-8) |w| and |mid| + |lo| <= 2^-7 |w|, the fp64
// additions (2^-40) and the fp32 stores of the partials (2^-23 of each),
//   |A - x.w| <= C1 sum_d |x_d w_d| + eta <= C1 ||x|| ||w|| + eta
// (Cauchy-Schwarz), with C1 = gamma_65 (1 + 2^-8) + gamma_129 2^-7
// + 1.02 2^-23 + 2^-40 and eta = 2^-123 (sqrt(D) (||x|| + ||w||) + D) for
// inputs, parts or products below the normal range that the matrix core may
// flush to zero. The logit compared is v = fl32(fl32(A) + bias) against the
// exact fl32(fl32(x.w) + bias); with the roundings of both,
//   |v - v_exact| <= eps = eraw + 2^-21 (2 |v| + |bias| + eraw).
//
// Certified top-k. Take the top-k of the approximate v (descending, ties to
// the lower id). If each chosen expert's v - eps exceeds the next chosen
// one's v + eps, and every expert not chosen has v + eps below the k-th
// chosen one's v - eps, the exact logits order the experts the same way and
// the choice is final. Otherwise the token's candidates are the chosen
// experts and every other expert whose v + eps is not below
// L = min over chosen j of (v_j - eps_j); their logits are recomputed exactly
// (exact products, fp64 sum, one rounding to fp32: the fp64 router's
// arithmetic) and the top-k is taken again over the row. Every expert left
// out has both its approximate and its exact logit below L, which every
// chosen expert's exact logit reaches, so the new choice is the one the
// exact logits give. Non-finite sums fail the tests (NaN compares false) and
// send the token down the exact path.
// ===========================================================================

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStep = 64;          // hidden elements per step
constexpr int kRowB = kStep * 2;   // bytes of one bf16 row of a step in LDS
constexpr int kSplitChunk = 1024;  // hidden elements per workgroup of the weight split
constexpr int kSelTok = 16;        // tokens per workgroup of the select kernel (8 for E > 512)

// Error constant of the approximate logits (see above).
__host__ __device__ constexpr double gamma_n(int n) {
  return n * 0x1p-23 / (1.0 - n * 0x1p-23);
}
constexpr double kC1 = (gamma_n(65) * (1.0 + 0x1p-8) + gamma_n(129) * 0x1p-7 + 1.02 * 0x1p-23 +
                        0x1p-40) * (1.0 + 0x1p-10);

// hi / mid / lo parts of four weights, as packed bf16 pairs.
__device__ __forceinline__ void split3(const uint4& raw, uint2& hi, uint2& mid, uint2& lo) {
  const float w[4] = {__uint_as_float(raw.x), __uint_as_float(raw.y), __uint_as_float(raw.z),
                      __uint_as_float(raw.w)};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 bh = static_cast<__bf16>(w[i]);
    const float r1 = w[i] - static_cast<float>(bh);
    const __bf16 bm = static_cast<__bf16>(r1);
    const float r2 = r1 - static_cast<float>(bm);
    const __bf16 bl = static_cast<__bf16>(r2);
    h[i] = __builtin_bit_cast(uint16_t, bh);
    m[i] = __builtin_bit_cast(uint16_t, bm);
    l[i] = __builtin_bit_cast(uint16_t, bl);
  }
  hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  mid = make_uint2(m[0] | (m[1] << 16), m[2] | (m[3] << 16));
  lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
}

// Weight split for E > 16: wsp [3][E][D] bf16 (hi, mid, lo) and the squared
// norm of each 1024-element piece of each row, wn2 [D / 1024][E] (fp64, exact
// squares). One workgroup per (row, piece); thread t handles 4 elements.
__global__ __launch_bounds__(kThreads) void route_split_weights_kernel(
    const float* __restrict__ wr, int D, int E, uint16_t* __restrict__ wsp,
    double* __restrict__ wn2) {
  __shared__ double red[kWaves];
  const int npc = (D + kSplitChunk - 1) / kSplitChunk;
  const int e = blockIdx.x / npc, pc = blockIdx.x % npc;
  const int k = pc * kSplitChunk + 4 * threadIdx.x;
  double s = 0.0;
  if (k < D) {
    const uint4 raw = *reinterpret_cast<const uint4*>(wr + static_cast<int64_t>(e) * D + k);
    uint2 hi, mid, lo;
    split3(raw, hi, mid, lo);
    const size_t plane = static_cast<size_t>(E) * D;
    const size_t o = static_cast<size_t>(e) * D + k;
    *reinterpret_cast<uint2*>(wsp + o) = hi;
    *reinterpret_cast<uint2*>(wsp + plane + o) = mid;
    *reinterpret_cast<uint2*>(wsp + 2 * plane + o) = lo;
    const double a = __uint_as_float(raw.x), b = __uint_as_float(raw.y),
                 c = __uint_as_float(raw.z), dd = __uint_as_float(raw.w);
    s = a * a + b * b + c * c + dd * dd;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) wn2[static_cast<int64_t>(pc) * E + e] = red[0] + red[1] + red[2] + red[3];
}

// Approximate partial logits of a TM-token x EN-expert tile over one slice of
// the hidden dimension. Waves WM x WN, each MT x NT blocks of 16 x 16.
// The weight parts come from route_split_weights_kernel. Grid: expert tiles
// fastest, then slices, then token tiles.
//   part [ksplit][T][E] fp32, xn2 [ksplit][T] fp64 (written by expert tile 0).
template <int MT, int NT, int WM, int WN>
__global__ __launch_bounds__(kThreads, 2) void route_gemm_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr,
    const uint16_t* __restrict__ wsp, int T, int D, int E, int n_et, int ksplit, int spk,
    float* __restrict__ part, double* __restrict__ xn2) {
  constexpr int TM = 16 * MT * WM, EN = 16 * NT * WN;
  constexpr int XB = TM * kRowB, WB = 3 * EN * kRowB, SB = XB + WB;
  constexpr int NXC = TM * 8 / kThreads;  // 16-byte x chunks per thread and step
  constexpr int NWQ = 3 * EN * 8;  // 16-byte weight chunks per step
  constexpr int NWC = (NWQ + kThreads - 1) / kThreads;
  static_assert(TM * 8 % kThreads == 0, "x tile must be whole chunks per thread");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b = blockIdx.x;
  const int et = b % n_et;
  b /= n_et;
  const int ks = b % ksplit, tt = b / ksplit;
  const int t0 = tt * TM, e0 = et * EN;
  const int s_begin = ks * spk, s_end = min(D / kStep, s_begin + spk);
  const bool do_xn = et == 0;

  // Two register sets of staged loads: the set of step i + 1 is written to
  // LDS during step i and refilled with step i + 3, so every load has two
  // steps to land.
  uint4 xr0[NXC], wg0[NWC], xr1[NXC], wg1[NWC];
  double xacc[NXC];
#pragma unroll
  for (int j = 0; j < NXC; ++j) xacc[j] = 0.0;

  // Every load is issued (rows past T or E read the last row; store() writes
  // zeros for them), so no branch or select waits on a load and the
  // compiler's count of loads in flight stays exact.
  auto load = [&](uint4 (&xr)[NXC], uint4 (&wg)[NWC], int s) {
    const int kb = s * kStep;
#pragma unroll
    for (int j = 0; j < NXC; ++j) {
      const int q = tid + kThreads * j, row = q >> 3, c = q & 7;
      xr[j] = *reinterpret_cast<const uint4*>(
          x + static_cast<int64_t>(min(t0 + row, T - 1)) * D + kb + 8 * c);
    }
#pragma unroll
    for (int j = 0; j < NWC; ++j) {
      const int q = min(tid + kThreads * j, NWQ - 1);
      const int sp = q / (EN * 8), r = q % (EN * 8), row = r >> 3, c = r & 7;
      wg[j] = *reinterpret_cast<const uint4*>(
          wsp + (static_cast<int64_t>(sp) * E + min(e0 + row, E - 1)) * D + kb + 8 * c);
    }
  };
  auto zero_if = [](const uint4& v, bool z) { return z ? make_uint4(0, 0, 0, 0) : v; };
  // Row r of a tile keeps its 16-byte chunk c at chunk c ^ (r & 7).
  // count: the stage holds a step of the slice (its squares enter the norms).
  auto store = [&](const uint4 (&xr)[NXC], const uint4 (&wg)[NWC], int st, bool count) {
    unsigned char* xs = lds + st * SB;
    unsigned char* ws = xs + XB;
#pragma unroll
    for (int j = 0; j < NXC; ++j) {
      const int q = tid + kThreads * j, row = q >> 3, c = q & 7;
      const uint4 xv = zero_if(xr[j], t0 + row >= T);
      *reinterpret_cast<uint4*>(xs + row * kRowB + ((c ^ (row & 7)) << 4)) = xv;
      if (do_xn && count) {
        const uint32_t u[4] = {xv.x, xv.y, xv.z, xv.w};
        float s2 = 0.f;  // squares of bf16 values are exact in fp32
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(u[i] << 16), hi = __uint_as_float(u[i] & 0xffff0000u);
          s2 = fmaf(lo, lo, s2);
          s2 = fmaf(hi, hi, s2);
        }
        xacc[j] += static_cast<double>(s2);
      }
    }
#pragma unroll
    for (int j = 0; j < NWC; ++j) {
      const int q = tid + kThreads * j;
      if (q >= NWQ) continue;
      const int sp = q / (EN * 8), r = q % (EN * 8), row = r >> 3, c = r & 7;
      *reinterpret_cast<uint4*>(ws + sp * EN * kRowB + row * kRowB + ((c ^ (row & 7)) << 4)) =
          zero_if(wg[j], e0 + row >= E);
    }
  };

  const int wm = wave % WM, wn = wave / WM;
  // Two accumulator sets, by step parity: the fp64 flush of one step's sums
  // runs while the next step's MFMAs write the other set.
  f32x4 acc_h[2][MT][NT], acc_m[2][MT][NT];
  double acc64[MT][NT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc64[m][n][i] = 0.0;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, auto par_c) {
    constexpr int P = decltype(par_c)::value;
    const unsigned char* xs = lds + st * SB;
    const unsigned char* ws = xs + XB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8 a[MT], w3[3][NT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int row = (wm * MT + m) * 16 + (lane & 15);
        a[m] = *reinterpret_cast<const bf16x8*>(xs + row * kRowB + ((c ^ (row & 7)) << 4));
      }
#pragma unroll
      for (int sp = 0; sp < 3; ++sp)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int row = (wn * NT + n) * 16 + (lane & 15);
          w3[sp][n] = *reinterpret_cast<const bf16x8*>(ws + sp * EN * kRowB + row * kRowB +
                                                       ((c ^ (row & 7)) << 4));
        }
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          acc_h[P][m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a[m], w3[0][n], kk == 0 ? zero : acc_h[P][m][n], 0, 0, 0);
          acc_m[P][m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a[m], w3[1][n], kk == 0 ? zero : acc_m[P][m][n], 0, 0, 0);
          acc_m[P][m][n] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], w3[2][n], acc_m[P][m][n], 0, 0, 0);
        }
    }
  };
  auto flush = [&](auto par_c) {
    constexpr int P = decltype(par_c)::value;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc64[m][n][i] +=
              static_cast<double>(acc_h[P][m][n][i]) + static_cast<double>(acc_m[P][m][n][i]);
  };

  // Two LDS stages. Step s_begin + i multiplies from stage i & 1 into
  // accumulator set i & 1 and flushes set (i - 1) & 1; the register set
  // holding step i + 1 is then stored to the other stage and refilled with
  // step i + 3. Loads and stores are issued on every pass (past the last
  // step they reload it and fill a stage no one reads), so no branch
  // surrounds them: the compiler then waits for one set only.
  const int n = s_end - s_begin;
  auto clamp_step = [&](int i) { return s_begin + min(i, n - 1); };
  load(xr0, wg0, s_begin);
  store(xr0, wg0, 0, true);
  load(xr1, wg1, clamp_step(1));
  load(xr0, wg0, clamp_step(2));
  __syncthreads();
  auto step = [&](int i, uint4 (&xr)[NXC], uint4 (&wg)[NWC], auto par_c) {
    constexpr int P = decltype(par_c)::value;  // == i & 1
    if (i < n) {
      compute(i & 1, par_c);
      if (i > 0) flush(std::integral_constant<int, P ^ 1>{});
    }
    store(xr, wg, (i + 1) & 1, i + 1 < n);
    load(xr, wg, clamp_step(i + 3));
    __syncthreads();
  };
  for (int i = 0; i < n; i += 2) {
    step(i, xr1, wg1, std::integral_constant<int, 0>{});
    step(i + 1, xr0, wg0, std::integral_constant<int, 1>{});
  }
  if ((n - 1) & 1)
    flush(std::integral_constant<int, 1>{});
  else
    flush(std::integral_constant<int, 0>{});

  // Output block of the 16x16 MFMA: lane l holds column l % 16 (expert) of
  // rows 4 (l / 16) + i (tokens).
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int e = e0 + (wn * NT + n) * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + (wm * MT + m) * 16 + 4 * (lane >> 4) + i;
        if (t < T && e < E)
          part[(static_cast<int64_t>(ks) * T + t) * E + e] = static_cast<float>(acc64[m][n][i]);
      }
    }
  if (do_xn) {
#pragma unroll
    for (int j = 0; j < NXC; ++j) {
      double v = xacc[j];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      const int q = tid + kThreads * j, t = t0 + (q >> 3);
      if ((q & 7) == 0 && t < T) xn2[static_cast<int64_t>(ks) * T + t] = v;
    }
  }
}

// Sum, in order, of p[0], p[stride], ..., p[(n - 1) stride]; the loads are
// issued four at a time before any of them is used.
template <typename T>
__device__ __forceinline__ double sum_strided(const T* __restrict__ p, int64_t stride, int n) {
  double s = 0.0;
  for (int i = 0; i < n; i += 4) {
    T v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[stride * min(i + u, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u < n) s += static_cast<double>(v[u]);
  }
  return s;
}


// The largest float below f (f finite).
__device__ __forceinline__ float next_down(float f) {
  if (f == 0.f) return -0x1p-149f;
  const uint32_t u = __float_as_uint(f);
  return __uint_as_float(f > 0.f ? u - 1 : u + 1);
}

// Group minimum of a float (every lane of the group ends with it).
template <int LPT>
__device__ __forceinline__ float group_min(float v) {
  int dummy = 0;
  float nv = -v;
  group_argmax<LPT>(nv, dummy);
  return -nv;
}

// Norms, rounded up: the sums of squares were formed with at most 2^-22
// relative error (fp32 sums of eight exact squares, fp64 beyond).
constexpr double kNormUp = 1.0 + 0x1p-20;

// LDS of the selection of TW tokens over E experts: nw [E] fp64 weight-row
// norms, nxs [TW] fp64 token norms, scal [2] fp64 (largest weight-row norm,
// largest finite |bias|), bs [E] bias (0 without), masks
// [TW][MOE_MAX_EXPERTS / 64] candidate bits, ls [TW][E] fp32 logits, then per
// token the candidate threshold, max, sum, the flagged list and its count,
// the chosen experts [TW][MOE_MAX_TOPK] and which of them need exact logits.
struct SelLds {
  double* nw;
  double* nxs;
  double* scal;
  float* bs;
  uint64_t* masks;
  float* ls;
  float* tok_L;
  float* tok_max;
  float* tok_sum;
  int* flagged;
  int* n_flag;
  int* chosen;
  uint32_t* needm;
};
__host__ __device__ inline size_t sel_lds_bytes(int E, int tw) {
  return static_cast<size_t>(E) * 8 + tw * 8 + 2 * 8 + (E + 1) / 2 * 8 +
         tw * (MOE_MAX_EXPERTS / 64) * 8 + static_cast<size_t>(tw) * E * 4 + 3 * tw * 4 +
         (tw + 1) * 4 + tw * MOE_MAX_TOPK * 4 + tw * 4;
}
__device__ inline SelLds sel_lds(unsigned char* base, int E, int tw) {
  SelLds L;
  L.nw = reinterpret_cast<double*>(base);
  L.nxs = L.nw + E;
  L.scal = L.nxs + tw;
  L.bs = reinterpret_cast<float*>(L.scal + 2);
  L.masks = reinterpret_cast<uint64_t*>(L.scal + 2 + (E + 1) / 2);
  L.ls = reinterpret_cast<float*>(L.masks + tw * (MOE_MAX_EXPERTS / 64));
  L.tok_L = L.ls + tw * E;
  L.tok_max = L.tok_L + tw;
  L.tok_sum = L.tok_max + tw;
  L.flagged = reinterpret_cast<int*>(L.tok_sum + tw);
  L.n_flag = L.flagged + tw;
  L.chosen = L.n_flag + 1;
  L.needm = reinterpret_cast<uint32_t*>(L.chosen + tw * MOE_MAX_TOPK);
  return L;
}

// Certified top-k of tokens t0 .. t0 + n_tok - 1 (see above), once the LDS
// holds their approximate logits (ls), the norms (nw, nxs), the bias (bs)
// and *n_flag = 0, behind a barrier: selection, candidate masks, exact
// logits of the candidates, selection again, outputs.
template <int LPT, int TW, int KPER>
__device__ void select_tile(const SelLds& L, const uint16_t* __restrict__ x,
                            const float* __restrict__ wr, const float* __restrict__ bias, int T,
                            int D, int E, int k, int norm_topk, int t0, int n_tok,
                            float* __restrict__ logits, float* __restrict__ probs,
                            int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int kPer = KPER;  // experts per lane: E <= LPT * KPER
  constexpr int kMaskWords = MOE_MAX_EXPERTS / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const double sqrt_d = sqrt(static_cast<double>(D));
  double* nw = L.nw;
  double* nxs = L.nxs;
  float* bs = L.bs;
  uint64_t* masks = L.masks;
  float* ls = L.ls;
  float* tok_L = L.tok_L;
  float* tok_max = L.tok_max;
  float* tok_sum = L.tok_sum;
  int* flagged = L.flagged;
  int* n_flag = L.n_flag;
  const int sub = lane / LPT, sl = lane % LPT;
  const int per_lane = (E + LPT - 1) / LPT;
  // The largest weight-row norm and the largest finite |bias| (NaN kept: it
  // fails every test below).
  if (wave == 0) {
    double mw = 0.0, mb = 0.0;
    for (int e = lane; e < E; e += 64) {
      const double a = nw[e], b = fabs(static_cast<double>(bs[e]));
      mw = (a > mw || a != a) ? a : mw;
      if (b != INFINITY) mb = (b > mb || b != b) ? b : mb;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double a = __shfl_xor(mw, off, 64), b = __shfl_xor(mb, off, 64);
      mw = (a > mw || a != a) ? a : mw;
      mb = (b > mb || b != b) ? b : mb;
    }
    if (lane == 0) {
      L.scal[0] = mw;
      L.scal[1] = mb;
    }
  }
  __syncthreads();
  const double nw_max = L.scal[0], b_max = L.scal[1];
  // k rounds of the group argmax over the row of token tk; lane j of the
  // group gets the j-th choice. Writes the outputs when `final`, else tests
  // the certificate and returns it (group-uniform).
  auto select = [&](int tk, bool valid, bool final) -> bool {
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
      if (j == 0) m = bv;
      s_sel += expf(bv - m);
      if (sl == j) { my_v = bv; my_e = be; }
      if (be % LPT == sl) taken |= 1u << (be / LPT);
    }
    bool ok = true;
    if (!final) {
      // One bound eps for all of the token's logits: the raw bound with the
      // largest weight-row norm, plus the fp32 roundings of values up to the
      // largest magnitude that can matter (the top choice, the k-th, and
      // 2 eps around them). Choices j and j + 1 are in certain order when
      // their approximate logits differ by more than 2 eps; the (k + 1)-th
      // is then below the k-th too.
      float v_next = -INFINITY;  // the best expert not chosen
      if (k < E) {  // (uniform)
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int e = sl + LPT * i;
          if (i < per_lane && e < E && !((taken >> i) & 1u)) take_better(bv, be, v[i], e);
        }
        group_argmax<LPT>(bv, be);
        v_next = bv;
      }
      const double nx = valid ? nxs[tk] : 0.0;
      const double er = kC1 * nx * nw_max + 0x1p-123 * (sqrt_d * (nx + nw_max) + D);
      const float vk = __shfl(my_v, sub * LPT + k - 1, 64);
      const double big = fmax(fabs(static_cast<double>(m)), fabs(static_cast<double>(vk))) + 4.0 * er;
      const double two_eps = 2.0 * (er + 0x1p-20 * (2.0 * big + b_max + er));
      const float v_up = __shfl(my_v, sl > 0 ? lane - 1 : lane, 64);
      const float v_dn_in = __shfl(my_v, sl + 1 < LPT ? lane + 1 : lane, 64);
      const float v_dn = sl + 1 < k ? v_dn_in : v_next;
      // Choices that need their exact logit: those within 2 eps of the
      // choice above or below (the k-th: of the best expert not chosen).
      bool need = false;
      if (sl < k && valid) {
        if (sl > 0 && !(static_cast<double>(v_up) - static_cast<double>(my_v) > two_eps))
          need = true;
        if (!(static_cast<double>(my_v) - static_cast<double>(v_dn) > two_eps)) need = true;
      }
      const uint64_t needs = __ballot(need);
      const uint32_t gneed = static_cast<uint32_t>(
          (needs >> (sub * LPT)) & (LPT == 64 ? ~0ull : ((1ull << LPT) - 1)));
      if (gneed != 0) {
        if (valid) {
          if (sl < k) L.chosen[tk * MOE_MAX_TOPK + sl] = my_e;
          if (sl == 0) {
            // Experts not chosen that may enter: approximate logit at least
            // the k-th's minus 2 eps (threshold rounded down to fp32).
            const double thr = static_cast<double>(vk) - two_eps;
            float tf = static_cast<float>(thr);
            if (static_cast<double>(tf) > thr) tf = next_down(tf);
            if (thr != thr) tf = -INFINITY;
            tok_L[tk] = tf;
            L.needm[tk] = gneed;
            flagged[atomicAdd(n_flag, 1)] = tk;
          }
        }
        return false;
      }
    }
    float s_all = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = sl + LPT * i;
      if (i < per_lane && e < E) s_all += expf(v[i] - m);
    }
    s_all = group_sum<LPT>(s_all);
    const float denom = norm_topk ? s_sel : s_all;
    if (valid) {
      const int64_t t = static_cast<int64_t>(t0) + tk;
      if (sl < k) {
        topk_idx[t * k + sl] = my_e;
        topk_w[t * k + sl] = expf(my_v - m) / denom;
      }
      if (sl == 0) {
        tok_max[tk] = m;
        tok_sum[tk] = s_all;
      }
    }
    return ok;
  };

  for (int tb = wave * (64 / LPT); tb < n_tok; tb += kWaves * (64 / LPT)) {
    const int tk = tb + sub;
    select(tk, tk < n_tok, false);
  }
  __syncthreads();
  const int nf = *n_flag;
  if (nf > 0) {  // (uniform)
    // Candidate masks of the flagged tokens: chunk c of 64 experts of
    // flagged token f is built by wave (f * words + c) % 4.
    const int words = (E + 63) / 64;
    for (int it = wave; it < nf * words; it += kWaves) {
      const int f = it / words, c = it % words, tk = flagged[f];
      const int e = c * 64 + lane;
      bool cand = false;
      if (e < E) {
        int slot = -1;
        for (int q = 0; q < k; ++q)
          if (L.chosen[tk * MOE_MAX_TOPK + q] == e) slot = q;
        cand = slot >= 0 ? ((L.needm[tk] >> slot) & 1u) != 0 : !(ls[tk * E + e] < tok_L[tk]);
      }
      const uint64_t mk = __ballot(cand);
      if (lane == 0) masks[f * kMaskWords + c] = mk;
    }
    __syncthreads();
    // Exact logits of the candidates: one wave per (token, expert) pair,
    // pairs dealt to the waves in order.
    int gi = 0;
    for (int f = 0; f < nf; ++f) {
      const int tk = flagged[f];
      const uint16_t* xp = x + (static_cast<int64_t>(t0) + tk) * D;
      for (int c = 0; c < words; ++c) {
        uint64_t mk = masks[f * kMaskWords + c];
        while (mk) {
          const int bit = __ffsll(static_cast<long long>(mk)) - 1;
          mk &= mk - 1;
          if ((gi++ % kWaves) != wave) continue;
          const int e = c * 64 + bit;
          const float* wp = wr + static_cast<int64_t>(e) * D;
          double s = 0.0;
          constexpr int kU = 8;  // 8-element chunks per lane with loads in flight
          for (int q0 = lane; q0 < D / 8; q0 += kU * 64) {
            uint4 xv[kU];
            float4 w0[kU], w1[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
              const int q = min(q0 + 64 * u, D / 8 - 1);
              xv[u] = *reinterpret_cast<const uint4*>(xp + 8 * q);
              w0[u] = *reinterpret_cast<const float4*>(wp + 8 * q);
              w1[u] = *reinterpret_cast<const float4*>(wp + 8 * q + 4);
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
              if (q0 + 64 * u >= D / 8) continue;  // (a clamped reload, not added)
              const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
              const float wv[8] = {w0[u].x, w0[u].y, w0[u].z, w0[u].w,
                                   w1[u].x, w1[u].y, w1[u].z, w1[u].w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                s = fma(static_cast<double>(__uint_as_float(xw[i] << 16)),
                        static_cast<double>(wv[2 * i]), s);
                s = fma(static_cast<double>(__uint_as_float(xw[i] & 0xffff0000u)),
                        static_cast<double>(wv[2 * i + 1]), s);
              }
            }
          }
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
          if (lane == 0) {
            float l = static_cast<float>(s);
            if (bias != nullptr) l += bs[e];
            if (l != l) l = -INFINITY;
            ls[tk * E + e] = l;
          }
        }
      }
    }
    __syncthreads();
    for (int fb = wave * (64 / LPT); fb < nf; fb += kWaves * (64 / LPT)) {
      const int f = fb + sub;
      const bool valid = f < nf;
      select(valid ? flagged[f] : 0, valid, true);
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


// Selection of a tile of TW tokens from the partial logits of
// route_gemm_kernel (see above).
template <int LPT, int TW, int KPER>
__global__ __launch_bounds__(kThreads) void route_select_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ part, int nparts, const double* __restrict__ xn2,
    const double* __restrict__ wn2, int nwp, int T, int D, int E, int k, int norm_topk,
    float* __restrict__ logits, float* __restrict__ probs, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const SelLds L = sel_lds(smem_raw, E, TW);
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TW;
  const int n_tok = min(TW, T - t0);
  if (tid == 0) *L.n_flag = 0;
  for (int e = tid; e < E; e += kThreads) {
    L.nw[e] = sqrt(sum_strided(wn2 + e, E, nwp)) * kNormUp;
    L.bs[e] = bias != nullptr ? bias[e] : 0.f;
  }
  for (int tk = tid; tk < n_tok; tk += kThreads)
    L.nxs[tk] = sqrt(sum_strided(xn2 + t0 + tk, T, nparts)) * kNormUp;
  for (int o = tid; o < n_tok * E; o += kThreads) {
    const int64_t g = static_cast<int64_t>(t0) * E + o;
    float l = static_cast<float>(sum_strided(part + g, static_cast<int64_t>(T) * E, nparts));
    if (bias != nullptr) l += bias[o % E];
    if (l != l) l = -INFINITY;  // a NaN logit is never preferred
    L.ls[o] = l;
  }
  __syncthreads();
  select_tile<LPT, TW, KPER>(L, x, wr, bias, T, D, E, k, norm_topk, t0, n_tok, logits, probs,
                             topk_idx, topk_w);
}

size_t select_lds_bytes(int E, int tw) { return sel_lds_bytes(E, tw); }

// Launch geometry and scratch layout of the bf16 router.
struct Bf16RoutePlan {
  int kind;   // 1: E <= 32 (tiles of 64 tokens x 32 experts); 2: 64 x 64
  int tm, en, n_tt, n_et, ksplit, spk, nwp;
  size_t part, xn2, wn2, wsp, total;
};

Bf16RoutePlan bf16_route_plan(int T, int D, int E) {
  Bf16RoutePlan p{};
  p.kind = E <= 32 ? 1 : 2;
  p.tm = 64;
  p.en = p.kind == 1 ? 32 : 64;
  p.n_tt = (T + p.tm - 1) / p.tm;
  p.n_et = (E + p.en - 1) / p.en;
  const int nsteps = D / kStep;
  // Slices of the hidden dimension until the grid has two workgroups per CU.
  const int64_t target = 512;
  int ks = 1;
  while (ks < 16 && ks * 2 <= nsteps && static_cast<int64_t>(p.n_tt) * p.n_et * ks < target)
    ks *= 2;
  p.spk = (nsteps + ks - 1) / ks;
  p.ksplit = (nsteps + p.spk - 1) / p.spk;
  p.nwp = (D + kSplitChunk - 1) / kSplitChunk;
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  size_t o = 0;
  p.part = o; o += al(static_cast<size_t>(p.ksplit) * T * E * 4);
  p.xn2 = o;  o += al(static_cast<size_t>(p.ksplit) * T * 8);
  p.wn2 = o;  o += al(static_cast<size_t>(p.nwp) * E * 8);
  p.wsp = o;  o += al(static_cast<size_t>(3) * E * D * 2);
  p.total = o;
  return p;
}

hipError_t launch_route_bf16(const moe_desc& d, const uint16_t* x, const float* wr,
                             const float* bias, float* logits, float* probs, int32_t* topk_idx,
                             float* topk_w, void* ws, hipStream_t s) {
  const Bf16RoutePlan p = bf16_route_plan(d.T, d.D, d.E);
  char* base = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(base + p.part);
  double* xn2 = reinterpret_cast<double*>(base + p.xn2);
  double* wn2 = reinterpret_cast<double*>(base + p.wn2);
  uint16_t* wsp = reinterpret_cast<uint16_t*>(base + p.wsp);
  const int grid = p.n_tt * p.n_et * p.ksplit;
#define MOE_GEMM_ARGS x, wr, wsp, d.T, d.D, d.E, p.n_et, p.ksplit, p.spk, part, xn2
  {
    const int npc = (d.D + kSplitChunk - 1) / kSplitChunk;
    route_split_weights_kernel<<<d.E * npc, kThreads, 0, s>>>(wr, d.D, d.E, wsp, wn2);
    if (p.kind == 1)
      route_gemm_kernel<2, 1, 2, 2><<<grid, kThreads, 0, s>>>(MOE_GEMM_ARGS);
    else
      route_gemm_kernel<2, 2, 2, 2><<<grid, kThreads, 0, s>>>(MOE_GEMM_ARGS);
  }
#undef MOE_GEMM_ARGS
  const int tw = d.E > 512 ? kSelTok / 2 : kSelTok;
  const int sgrid = (d.T + tw - 1) / tw;
  const size_t lds = select_lds_bytes(d.E, tw);
#define MOE_SEL_ARGS                                                                       \
  x, wr, bias, part, p.ksplit, xn2, wn2, p.nwp, d.T, d.D, d.E, d.top_k, d.norm_topk, logits, \
      probs, topk_idx, topk_w
  // Sixteen lanes per token (four tokens of a wave side by side) up to 256
  // experts; with 64 lanes per token the k argmax rounds of each token ran
  // one after another through the whole wave.
  if (d.E <= 32)
    route_select_kernel<16, kSelTok, 2><<<sgrid, kThreads, lds, s>>>(MOE_SEL_ARGS);
  else if (d.E <= 64)
    route_select_kernel<16, kSelTok, 4><<<sgrid, kThreads, lds, s>>>(MOE_SEL_ARGS);
  else if (d.E <= 128)
    route_select_kernel<16, kSelTok, 8><<<sgrid, kThreads, lds, s>>>(MOE_SEL_ARGS);
  else if (d.E <= 256)
    route_select_kernel<16, kSelTok, 16><<<sgrid, kThreads, lds, s>>>(MOE_SEL_ARGS);
  else if (d.E <= 512)
    route_select_kernel<32, kSelTok, 16><<<sgrid, kThreads, lds, s>>>(MOE_SEL_ARGS);
  else
    route_select_kernel<64, kSelTok / 2, 16><<<sgrid, kThreads, lds, s>>>(MOE_SEL_ARGS);
#undef MOE_SEL_ARGS
  return hipGetLastError();
}

}  // namespace

// bf16 activations with more than 16 experts take the bf16-split path; with
// at most 16 the fp64 router is the faster (its fp64 work is small there).
bool use_bf16_route(const moe_desc& d) { return d.act_dtype == MOE_BF16 && d.E > 16; }

size_t route_ws_bytes(const moe_desc& d) {
  if (!use_bf16_route(d) || d.T == 0) return 0;
  return bf16_route_plan(d.T, d.D, d.E).total;
}

hipError_t launch_route(const moe_desc& d, const void* x, const float* w_router,
                        const float* bias, float* logits, float* probs, int32_t* topk_idx,
                        float* topk_w, void* ws, hipStream_t s) {
  if (use_bf16_route(d))
    return launch_route_bf16(d, static_cast<const uint16_t*>(x), w_router, bias, logits, probs,
                             topk_idx, topk_w, ws, s);
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
