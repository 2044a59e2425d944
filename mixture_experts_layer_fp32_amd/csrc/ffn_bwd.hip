// Grouped GEMMs of the expert FFN's backward pass for bf16 layers, on gfx950
// matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// The forward is the SiLU-gated two-layer FFN of each expert (page "Expert
// Parallel (EP)", Communication Pattern stage 3 and Requirements; page
// "Worked Example", Step 3): G | U = X Wgu, H = SiLU(G) U, Y = H Wd. Its
// gradients, per expert segment of rows:
//   dH  = dY Wd^T                      (NT: both operands K-contiguous; fp32)
//   dG  = dH U SiLU'(G), dU = dH SiLU(G), and H    (epilogue of the forward
//                                       gate_up GEMM, which recomputes G and
//                                       U in its fp32 accumulators; or, when
//                                       the training forward saved G | U in
//                                       fp32, epilogue of the dH GEMM)
//   dX  = [dG | dU] Wgu^T              (NT)
//   dWd = H^T dY,  dWgu = X^T [dG | dU]   (TN: the contraction runs over the
//                                       segment's rows)
//
// NT kernel. C[r, c] = sum_k A[r, k] W_e[c, k]: the weight of expert e is read
// as [N_out rows][K] (down_proj [I, D] for dH, gate_up_proj [D, 2I] for dX),
// so both operands are staged and read like the forward's activations:
// 128-byte LDS rows (64 bf16 of K), 16-byte chunk c of row r at
// c ^ (r & 7) ^ ((r >> 3) & 1), one ds_read_b128 per fragment. Tiles of
// 320 rows x 128 columns, 4 waves (wave (wm, wn): 160 rows x 64 columns, 5 x 2
// blocks of 32 x 32), one workgroup per CU working through the tile list in
// XCD runs (as the forward's narrow tiles); activations one K-step ahead (2
// slots), weights two (3 slots), copies with the buffer-load-to-LDS path.
//
// TN kernel. C_e[p, q] = sum_{m in segment e} A[m, p] B[m, q], fp32 out, one
// 128 x 256 tile per workgroup (wave: 64 x 128, 2 x 4 blocks), two
// workgroups per CU. Both operands are [rows][columns] in memory with the
// contraction over rows, so both are staged like the forward's weights
// ([k][columns] x 16-bit, chunk c of row k at c ^ 4 (k & 3)) and read with
// two ds_read_b64_tr_b16 per fragment. Rows past the segment read as zeros;
// an expert without rows gets a zero gradient.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kMaxTableExperts = MOE_MAX_EXPERTS;
// A load offset past every buffer: the host keeps every operand below 2^30
// bytes, and offset + step offset stays below 2^32.
constexpr int kOutOfRange = 0x7FFF0000;

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes global -> LDS at lds_base + 16 * lane (M0 holds the LDS base).
// Out-of-range offsets write zeros. Counted by vmcnt.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff,
                                      unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// 4x4 transpose inside each group of 4 lanes: accumulator register r of lane
// l holds row 8 (r / 4) + 4 (l / 32) + r % 4 and column l % 32 of its 32x32
// block; after the transpose of registers 4g .. 4g + 3, lane l holds columns
// 4 (l % 32 / 4) .. + 3 of row 8 g + 4 (l / 32) + l % 4.
__device__ __forceinline__ void transpose4(float (&v)[4], int quad) {
  float n[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float x = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[r ^ 1]), 0xB1, 0xF, 0xF, false));
    n[r] = ((r ^ quad) & 1) ? x : v[r];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float x = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, n[r ^ 2]), 0x4E, 0xF, 0xF, false));
    v[r] = ((r ^ quad) & 2) ? x : n[r];
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16(a) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// ===========================================================================
// NT: grouped over expert segments of rows
// ===========================================================================
namespace nt {
constexpr int BM = 320;          // rows per tile
constexpr int kMaxMB = 5;        // 32-row blocks per wave row
constexpr int WN = 64;           // columns per wave
constexpr int NQ = 2;            // 32-column blocks per wave
constexpr int BN = 2 * WN;       // columns per tile (weight rows)
constexpr int BK = 64;           // K per step (128 bytes per row)
constexpr int kTileA = BM * 128;
constexpr int kTileB = BN * 128;
constexpr int NSB = 3;
constexpr int NA = BM / 32;      // 1 KB activation copies per wave per step
constexpr int NB = BN / 32;      // 1 KB weight copies per wave per step
}  // namespace nt

__device__ __forceinline__ int a_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int a_off(int row, int chunk) {
  return row * 128 + ((chunk ^ a_swz(row)) << 4);
}

enum NtEpilogue { kStoreF32 = 0, kSwigluSaved = 1 };

// kStoreF32: C [cap, N_out] fp32: row r of expert e's segment times W_e^T.
// kSwigluSaved: C = dH [rows, N_out = I]; gu holds the forward's G | U
//   [cap, 2 I] (fp32); writes dgu = dG | dU [cap, 2 I] and h [cap, I]
//   (bf16). The G | U values of a 32-row block are loaded while the previous
//   block is computed (those of the first block before the K loop).
template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_bf16(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int n_experts,
    int64_t cap_rows, const uint16_t* __restrict__ W, int K, int N_out, float* __restrict__ cf,
    const float* __restrict__ gu, uint16_t* __restrict__ dgu, uint16_t* __restrict__ hout) {
  using namespace nt;
  constexpr int kLds = 2 * kTileA + NSB * kTileB;
  static_assert(kLds + 2 * (kMaxTableExperts + 1) * 4 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLds];
  __shared__ int s_tab[2 * (kMaxTableExperts + 1)];
  int* s_pref = s_tab;                        // tiles before expert e
  int* s_off = s_tab + kMaxTableExperts + 1;  // first row of expert e (clamped to cap)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = (N_out + BN - 1) / BN;
  const int nk = K / BK;
  const int n_exp = offsets ? n_experts : 1;

  // ---- tile table: per-expert prefix of tile counts ----
  if (wave == 0) {
    const int lane = tid & 63;
    int base = 0;
    for (int e0 = 0; e0 < n_exp; e0 += 64) {
      const int e = e0 + lane;
      int beg = 0, end = 0;
      if (e < n_exp) {
        if (offsets) {
          beg = offsets[e];
          end = offsets[e + 1];
        } else {
          end = static_cast<int>(cap_rows);
        }
        beg = static_cast<int>(min(max(static_cast<int64_t>(beg), int64_t(0)), cap_rows));
        end = static_cast<int>(
            min(max(static_cast<int64_t>(end), static_cast<int64_t>(beg)), cap_rows));
      }
      const int tiles = ((end - beg + BM - 1) / BM) * NT;
      int incl = tiles;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      if (e < n_exp) {
        s_pref[e] = base + incl - tiles;
        s_off[e] = beg;
        if (e == n_exp - 1) {
          s_pref[n_exp] = base + incl;
          s_off[n_exp] = end;
        }
      }
      base += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  const int R = __builtin_amdgcn_readfirstlane(s_pref[n_exp]);
  const int G8 = static_cast<int>(gridDim.x) / kXcds;
  const int xcd = static_cast<int>(blockIdx.x) % kXcds, slot = static_cast<int>(blockIdx.x) / kXcds;
  const int per = (R + kXcds - 1) / kXcds;
  const int run_end = min((xcd + 1) * per, R);
  for (int t = xcd * per + slot; t < run_end; t += G8) {
    // Lane-derived values are computed per tile (not hoisted out of the loop).
    int lane_t = tid & 63;
    asm volatile("" : "+v"(lane_t));
    const int lane = lane_t;

    int expert = 0;
    for (int e0 = 1; e0 <= n_exp; e0 += 64) {
      const int idx = e0 + lane;
      const bool le = idx <= n_exp && s_pref[idx] <= t;
      expert += __popcll(__ballot(le));
      if (__ballot(idx <= n_exp && !le)) break;
    }
    expert = __builtin_amdgcn_readfirstlane(expert);
    const int seg_beg = __builtin_amdgcn_readfirstlane(s_off[expert]);
    const int seg_end = __builtin_amdgcn_readfirstlane(s_off[expert + 1]);
    const int local = t - __builtin_amdgcn_readfirstlane(s_pref[expert]);
    const int cnt = seg_end - seg_beg;
    const int mt = (cnt + BM - 1) / BM;
    const int chunk = (cnt + mt - 1) / mt;
    const int nb = local / mt, mbk = local - nb * mt;
    const int row_begin = seg_beg + mbk * chunk;
    const int rows = min(chunk, seg_end - row_begin);  // <= BM
    if (rows <= 0) continue;  // (uniform)
    const int n0 = nb * BN;

    // ---- copies (global -> LDS) ----
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + static_cast<int64_t>(row_begin) * K), 0, rows * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + static_cast<int64_t>(expert) * N_out * K), 0, N_out * K * 2, 0x00020000);
    int a_voff[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = 8 * (wave * NA + i) + (lane >> 3);
      a_voff[i] = row < rows ? row * K * 2 + (((lane & 7) ^ a_swz(row)) << 4) : kOutOfRange;
    }
    int b_voff[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = 8 * (wave * NB + i) + (lane >> 3);
      b_voff[i] = n0 + j < N_out ? (n0 + j) * K * 2 + (((lane & 7) ^ a_swz(j)) << 4)
                                 : kOutOfRange;
    }
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_u8*)smem;

    // ---- compute assignment: wave (wm, wn) ----
    const int wm = wave >> 1, wn = wave & 1;
    const int nblk = (rows + 31) / 32;
    const int nmb = wm == 0 ? (nblk + 1) / 2 : nblk / 2;
    const int rowbase = wm == 0 ? 0 : 32 * ((nblk + 1) / 2);
    const int half = lane >> 5;
    // Fragment of K-slice kk: chunk 2 kk + half of the row (K values
    // 16 kk + 8 half .. + 7), for the activation row and the weight row alike.
    int a_addr[4], b_addr[NQ][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      a_addr[kk] = a_off(rowbase + (lane & 31), 2 * kk + half);
#pragma unroll
      for (int q = 0; q < NQ; ++q) b_addr[q][kk] = a_off(wn * WN + q * 32 + (lane & 31), 2 * kk + half);
    }

    f32x16 acc[kMaxMB][NQ];
#pragma unroll
    for (int mb = 0; mb < kMaxMB; ++mb)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][q][r] = 0.f;

    // A copy that is not needed (a step past the last) is still issued, with
    // an out-of-range offset (it reads nothing and writes zeros into a
    // finished step's slot), so the K loop has no branch around it.
    auto copy_item = [&](int i, bool do_a, int kt_a, int slot_a, bool do_b, int kt_b,
                         int slot_b) {
      if (i < NA) {
        dma16(a_rsrc, do_a ? a_voff[i] : kOutOfRange, kt_a * BK * 2,
              lds0 + slot_a * kTileA + (wave * NA + i) * 1024);
      } else if (i - NA < NB) {
        dma16(b_rsrc, do_b ? b_voff[i - NA] : kOutOfRange, kt_b * BK * 2,
              lds0 + 2 * kTileA + slot_b * kTileB + (wave * NB + i - NA) * 1024);
      }
    };

    auto run = [&](auto nmb_c) {
      constexpr int NMB = decltype(nmb_c)::value;
      auto load = [&](int sa, int sb, int kk, uint4(&fa)[kMaxMB], uint4(&fb)[NQ]) {
        const unsigned char* abase = smem + sa * kTileA;
        const unsigned char* bbase = smem + 2 * kTileA + sb * kTileB;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          fa[mb] = *reinterpret_cast<const uint4*>(abase + a_addr[kk] + mb * 32 * 128);
#pragma unroll
        for (int q = 0; q < NQ; ++q) fb[q] = *reinterpret_cast<const uint4*>(bbase + b_addr[q][kk]);
      };
      // Prologue: weights of steps 0 and 1, activations of step 0.
#pragma unroll
      for (int i = NA; i < NA + NB; ++i) copy_item(i, false, 0, 0, true, 0, 0);
#pragma unroll
      for (int i = 0; i < NA + NB; ++i) copy_item(i, true, 0, 0, nk > 1, 1, 1);
      int sb = 0;
      for (int kt = 0; kt < nk; ++kt) {
        const int sa = kt & 1;
        // This wave's copies of step kt are done (only the weight copies of
        // step kt + 1 may be in flight); after the barrier every wave's are,
        // and every wave is done with step kt - 1's slots.
        if (kt + 1 < nk)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(NB));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
        const bool do_a = kt + 1 < nk, do_b = kt + 2 < nk;
        const int slot_a = sa ^ 1, slot_b = sb == 0 ? NSB - 1 : sb - 1;
        uint4 fa[2][kMaxMB], fb[2][NQ];
        if (NMB > 0) load(sa, sb, 0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (NMB > 0 && kk < 3) load(sa, sb, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mb = 0; mb < kMaxMB; ++mb) {
            if (mb < NMB) {
#pragma unroll
              for (int q = 0; q < NQ; ++q)
                acc[mb][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, fa[kk & 1][mb]),
                    __builtin_bit_cast(bf16x8, fb[kk & 1][q]), acc[mb][q], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            copy_item(kk * kMaxMB + mb, do_a, kt + 1, slot_a, do_b, kt + 2, slot_b);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        sb = sb == NSB - 1 ? 0 : sb + 1;
      }
    };
    // kSwigluSaved: G | U of row block mb (columns of this lane after the
    // epilogue's transpose), loaded ahead of their use.
    constexpr int NQE = EPI == kSwigluSaved ? NQ : 1;
    float4 gpre[2][NQE][4], upre[2][NQE][4];
    auto load_gu = [&](int mb, float4(&gq)[NQE][4], float4(&uq)[NQE][4]) {
#pragma unroll
      for (int q = 0; q < NQE; ++q) {
        const int col = n0 + wn * WN + q * 32 + (lane & 28);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = row_begin + rowbase + mb * 32 + 8 * g + 4 * half + (lane & 3);
          const bool ok = row < row_begin + rows && col < N_out;
          const int64_t gi = static_cast<int64_t>(row) * 2 * N_out + col;
          gq[q][g] = ok ? *reinterpret_cast<const float4*>(gu + gi) : make_float4(0.f, 0.f, 0.f, 0.f);
          uq[q][g] = ok ? *reinterpret_cast<const float4*>(gu + gi + N_out)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    };
    if (EPI == kSwigluSaved && nmb > 0) load_gu(0, gpre[0], upre[0]);
    static_assert(NA + NB <= 4 * kMaxMB, "copy items fit the MFMA groups");
    switch (nmb) {
      case 5: run(std::integral_constant<int, 5>{}); break;
      case 4: run(std::integral_constant<int, 4>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      default: run(std::integral_constant<int, 0>{}); break;
    }
    if (nmb > 0) {
      const int quad = lane & 3;
      const int row_end = row_begin + rows;
#pragma unroll
      for (int mb = 0; mb < kMaxMB; ++mb) {
        if (mb >= nmb) break;
        if (EPI == kSwigluSaved && mb + 1 < nmb)
          load_gu(mb + 1, gpre[(mb + 1) & 1], upre[(mb + 1) & 1]);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int col = n0 + wn * WN + q * 32 + (lane & 28);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[mb][q][4 * g + i];
            transpose4(v, quad);
            const int row = row_begin + rowbase + mb * 32 + 8 * g + 4 * half + quad;
            if (row >= row_end || col >= N_out) continue;
            if (EPI == kStoreF32) {
              *reinterpret_cast<float4*>(cf + static_cast<int64_t>(row) * N_out + col) =
                  make_float4(v[0], v[1], v[2], v[3]);
              continue;
            }
            // SiLU(g) = g s, s = 1 / (1 + exp(-g)); SiLU'(g) = s + SiLU(g) (1 - s).
            const float4 g4 = gpre[mb & 1][q < NQE ? q : 0][g];
            const float4 u4 = upre[mb & 1][q < NQE ? q : 0][g];
            const float gs[4] = {g4.x, g4.y, g4.z, g4.w}, us[4] = {u4.x, u4.y, u4.z, u4.w};
            float dg[4], du[4], hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sg =
                  __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gs[i]));
              const float silu = gs[i] * sg;
              dg[i] = v[i] * us[i] * (sg + silu * (1.f - sg));
              du[i] = v[i] * silu;
              hv[i] = silu * us[i];
            }
            const int64_t gi = static_cast<int64_t>(row) * 2 * N_out + col;
            *reinterpret_cast<uint2*>(dgu + gi) =
                make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
            *reinterpret_cast<uint2*>(dgu + gi + N_out) =
                make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
            *reinterpret_cast<uint2*>(hout + static_cast<int64_t>(row) * N_out + col) =
                make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          }
        }
      }
    }
    // Every wave is done with this tile's LDS before the next tile's copies.
    __syncthreads();
  }
}

// ===========================================================================
// TN: weight gradients, contraction over each expert's rows
// ===========================================================================
// TN tile shapes. Wave (wm, wn) of the 2 x 2 layout owns BP / 2 rows (p) and
// BQ / 2 columns (q) of the BP x BQ tile; both operands are staged as BK rows
// (k) of BP (resp. BQ) 16-bit values in NS ring slots.
template <int BP_, int BQ_, int BK_, int NS_>
struct TnShape {
  static constexpr int BP = BP_, BQ = BQ_, BK = BK_, NS = NS_;
  static constexpr int ROWA = BP * 2, ROWB = BQ * 2;  // bytes per staged row
  static constexpr int TILE_A = BK * ROWA, TILE_B = BK * ROWB;
  static constexpr int NCA = TILE_A / 4096, NCB = TILE_B / 4096;  // 1 KB copies per wave
  static constexpr int NCI = NCA + NCB;                           // copies per wave per step
  static constexpr int MP = BP / 64, MQ = BQ / 64;  // 32-blocks per wave, each way
  static constexpr int NKK = BK / 16;               // K-slices per step
  static constexpr int LDS = NS * (TILE_A + TILE_B);
  static_assert(TILE_A % 4096 == 0 && TILE_B % 4096 == 0, "whole copies per wave");
  static_assert(ROWA >= 256 && ROWB >= 256, "the chunk swizzle needs 16 chunks per row");
  static_assert(NS >= 2 && NCI * (NS - 2) < 64, "vmcnt counts the copies in flight");
};
// 128 x 256 tiles, 3 ring slots of 32-row steps (72 KB of LDS, 128
// accumulators per wave): two workgroups per CU, so one's fp32 gradient
// stores overlap the other's K loop.
using TnPair = TnShape<128, 256, 32, 3>;
constexpr int kTnBlocksPerCu = 2;

// LDS byte offset of element (k, col) of a staged tile with `row` bytes per
// row: 16-byte chunk col / 8 at position (col / 8) ^ 4 (k & 3).
__device__ __forceinline__ int t_off(int row, int k, int col) {
  return k * row + (((col >> 3) ^ ((k & 3) << 2)) << 4) + ((col & 7) << 1);
}

template <class S, int MINB>
__global__ __launch_bounds__(kThreads, MINB) void gemm_tn_bf16(
    const uint16_t* __restrict__ A, int P, const uint16_t* __restrict__ B, int Q,
    const int32_t* __restrict__ offsets, int n_experts, int64_t cap_rows,
    float* __restrict__ C) {
  constexpr int BP = S::BP, BQ = S::BQ, BK = S::BK, NS = S::NS;
  constexpr int ROWA = S::ROWA, ROWB = S::ROWB, NCA = S::NCA, NCB = S::NCB, NCI = S::NCI;
  constexpr int MP = S::MP, MQ = S::MQ, NKK = S::NKK;
  constexpr int CHA = ROWA / 16, CHB = ROWB / 16;     // chunks per staged row
  constexpr int RPA = 1024 / ROWA, RPB = 1024 / ROWB;  // staged rows per copy
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S::LDS];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int TP = (P + BP - 1) / BP, TQ = (Q + BQ - 1) / BQ;
  // Every XCD takes an eighth of every expert's tiles (local tile li = p
  // block * TQ + q block with li = x mod 8 on XCD x), expert by expert: the
  // experts' row counts (the K loops) can differ widely, and this keeps the
  // XCDs' shares of the work equal; the eight XCDs work on the same expert at
  // the same time, so its operands are fetched from HBM into the shared
  // last-level cache about once. Workgroup b runs on XCD b mod 8.
  const int TPQ = TP * TQ;
  const int x = static_cast<int>(blockIdx.x) % kXcds, tx = static_cast<int>(blockIdx.x) / kXcds;
  const int nx = (TPQ - x + kXcds - 1) / kXcds;  // tiles of one expert on XCD x
  if (nx == 0 || tx >= nx * n_experts) return;
  const int e = tx / nx;
  const int li = kXcds * (tx - e * nx) + x;
  const int p0 = (li / TQ) * BP, q0 = (li % TQ) * BQ;
  int64_t beg = 0, end = cap_rows;
  if (offsets) {
    beg = min(max(static_cast<int64_t>(offsets[e]), int64_t(0)), cap_rows);
    end = min(max(static_cast<int64_t>(offsets[e + 1]), beg), cap_rows);
  }
  const int cnt = __builtin_amdgcn_readfirstlane(static_cast<int>(end - beg));
  const int nk = (cnt + BK - 1) / BK;

  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + beg * P), 0, cnt * P * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + beg * Q), 0, cnt * Q * 2, 0x00020000);
  // Copy i of a wave fills 1 KB of the slot: staged rows RP (NC wave + i) ..
  // + RP - 1; lane -> row + lane / CH, LDS chunk lane % CH (the global chunk
  // swizzled, so that LDS chunk s of row k holds global chunk s ^ 4 (k & 3)).
  int a_voff[NCA], b_voff[NCB];
#pragma unroll
  for (int i = 0; i < NCA; ++i) {
    const int k = RPA * (NCA * wave + i) + lane / CHA;
    const int c = 8 * ((lane % CHA) ^ ((k & 3) << 2));
    a_voff[i] = p0 + c < P ? (k * P + p0 + c) * 2 : kOutOfRange;
  }
#pragma unroll
  for (int i = 0; i < NCB; ++i) {
    const int k = RPB * (NCB * wave + i) + lane / CHB;
    const int c = 8 * ((lane % CHB) ^ ((k & 3) << 2));
    b_voff[i] = q0 + c < Q ? (k * Q + q0 + c) * 2 : kOutOfRange;
  }
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_u8*)smem;
  // Slot s: A tile at s * TILE_A, B tile at NS * TILE_A + s * TILE_B.
  auto copy_item = [&](int i, int kt, int slot) {
    if (i < NCA)
      dma16(a_rsrc, a_voff[i], kt * BK * P * 2,
            lds0 + slot * S::TILE_A + (wave * NCA + i) * 1024);
    else
      dma16(b_rsrc, b_voff[i - NCA], kt * BK * Q * 2,
            lds0 + NS * S::TILE_A + slot * S::TILE_B + (wave * NCB + i - NCA) * 1024);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int grp = lane >> 4, j16 = lane & 15;
  // Fragment of a 32-block at column blk: lane j of 16-lane group g reads 8
  // bytes of staged row 8 (g >> 1) + (j >> 2) (and + 4) at column
  // blk + 16 (g & 1) + 4 (j & 3): lane l then holds K-values 8 (l >> 5) .. + 7
  // of column blk + l % 32.
  int fa_addr[MP], fb_addr[MQ];
#pragma unroll
  for (int i = 0; i < MP; ++i)
    fa_addr[i] = t_off(ROWA, 8 * (grp >> 1) + (j16 >> 2),
                       wm * (BP / 2) + 32 * i + 16 * (grp & 1) + 4 * (j16 & 3));
#pragma unroll
  for (int j = 0; j < MQ; ++j)
    fb_addr[j] = t_off(ROWB, 8 * (grp >> 1) + (j16 >> 2),
                       wn * (BQ / 2) + 32 * j + 16 * (grp & 1) + 4 * (j16 & 3));

  f32x16 acc[MP][MQ];
#pragma unroll
  for (int i = 0; i < MP; ++i)
#pragma unroll
    for (int j = 0; j < MQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto frag = [&](const lds_u8* p, int row) {
    const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
    const uint2 hi = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * row)));
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  auto load = [&](int slot, int kk, uint4(&fa)[MP], uint4(&fb)[MQ]) {
    const lds_u8* abase = (const lds_u8*)smem + slot * S::TILE_A + kk * 16 * ROWA;
    const lds_u8* bbase = (const lds_u8*)smem + NS * S::TILE_A + slot * S::TILE_B + kk * 16 * ROWB;
#pragma unroll
    for (int i = 0; i < MP; ++i) fa[i] = frag(abase + fa_addr[i], ROWA);
#pragma unroll
    for (int j = 0; j < MQ; ++j) fb[j] = frag(bbase + fb_addr[j], ROWB);
  };

  // Steps 0 .. NS - 2 in flight before the loop; step kt + NS - 1 is copied
  // during step kt into the slot step kt - 1 used.
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) {
#pragma unroll
      for (int i = 0; i < NCI; ++i) copy_item(i, st, st);
    }
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // This wave's copies of step kt are done (copies complete in order; those
    // of the later steps in flight may remain); after the barrier every
    // wave's are, and every wave is done reading step kt - 1.
    if (NS > 2 && kt + 1 < nk)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NCI * (NS - 2)));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    const int kn = kt + NS - 1;  // step copied during this one
    const bool more = kn < nk;
    const int nslot = slot == 0 ? NS - 1 : slot - 1;  // = kn mod NS
    uint4 fa[2][MP], fb[2][MQ];
    load(slot, 0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk + 1 < NKK) load(slot, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MP; ++i) {
#pragma unroll
        for (int j = 0; j < MQ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, fa[kk & 1][i]), __builtin_bit_cast(bf16x8, fb[kk & 1][j]),
              acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // the step's copies spread over its NKK * MP groups of MFMAs
        const int grp_i = kk * MP + i;
        if (more) {
#pragma unroll
          for (int c = 0; c < NCI; ++c)
            if (c * (NKK * MP) / NCI == grp_i) copy_item(c, kn, nslot);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    slot = slot + 1 == NS ? 0 : slot + 1;
  }

  // ---- epilogue: fp32 gradient tile ----
  const int quad = lane & 3, half = lane >> 5;
  float* Ce = C + static_cast<int64_t>(e) * P * Q;
#pragma unroll
  for (int i = 0; i < MP; ++i) {
#pragma unroll
    for (int j = 0; j < MQ; ++j) {
      const int q = q0 + wn * (BQ / 2) + j * 32 + (lane & 28);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r];
        transpose4(v, quad);
        const int p = p0 + wm * (BP / 2) + i * 32 + 8 * g + 4 * half + quad;
        if (p < P && q < Q)
          *reinterpret_cast<float4*>(Ce + static_cast<int64_t>(p) * Q + q) =
              make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

int num_cus_bwd() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess)
      cus = p.multiProcessorCount;
    if (cus <= 0) cus = 256;
  }
  return cus;
}

template <int EPI>
hipError_t launch_nt(int n_experts, int64_t cap_rows, int K, int n_out, const void* a,
                     const int32_t* offsets, const void* w, float* cf, hipStream_t s,
                     const float* gu = nullptr, void* dgu = nullptr, void* h = nullptr) {
  using namespace nt;
  const int64_t mtiles = (cap_rows + BM - 1) / BM + (offsets ? n_experts : 0);
  const int64_t tiles = mtiles * ((n_out + BN - 1) / BN);
  const int64_t cus = std::max<int64_t>(kXcds, num_cus_bwd() / kXcds * kXcds);
  const int64_t g = std::min((tiles + kXcds - 1) / kXcds * kXcds, cus);
  gemm_nt_bf16<EPI><<<static_cast<unsigned>(g), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(a), offsets, n_experts, cap_rows,
      static_cast<const uint16_t*>(w), K, n_out, cf, gu, static_cast<uint16_t*>(dgu),
      static_cast<uint16_t*>(h));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dh_bwd(int n_experts, int64_t cap_rows, int D, int inter, const void* dy_perm,
                         const int32_t* offsets, const void* w_down, float* dh, hipStream_t s) {
  if (cap_rows == 0) return hipSuccess;
  return launch_nt<kStoreF32>(n_experts, cap_rows, D, inter, dy_perm, offsets, w_down, dh, s);
}

hipError_t launch_dh_swiglu_saved(int n_experts, int64_t cap_rows, int D, int inter,
                                  const void* dy_perm, const int32_t* offsets,
                                  const void* w_down, const float* gu, void* dgu, void* h,
                                  hipStream_t s) {
  if (cap_rows == 0) return hipSuccess;
  return launch_nt<kSwigluSaved>(n_experts, cap_rows, D, inter, dy_perm, offsets, w_down,
                                 nullptr, s, gu, dgu, h);
}

hipError_t launch_dx_perm_bwd(int n_experts, int64_t cap_rows, int D, int inter, const void* dgu,
                              const int32_t* offsets, const void* w_gate_up, float* dx_perm,
                              hipStream_t s) {
  if (cap_rows == 0) return hipSuccess;
  return launch_nt<kStoreF32>(n_experts, cap_rows, 2 * inter, D, dgu, offsets, w_gate_up,
                              dx_perm, s);
}

hipError_t launch_wgrad_bf16(int n_experts, int64_t cap_rows, const void* a, int P, const void* b,
                             int Q, const int32_t* offsets, float* c, hipStream_t s) {
  using S = TnPair;
  const int64_t tpq = static_cast<int64_t>((P + S::BP - 1) / S::BP) * ((Q + S::BQ - 1) / S::BQ);
  if (tpq == 0 || n_experts == 0) return hipSuccess;
  // XCD 0 has the most tiles per expert: ceil(tpq / 8)
  const int64_t g = (tpq + kXcds - 1) / kXcds * n_experts * kXcds;
  gemm_tn_bf16<S, kTnBlocksPerCu><<<static_cast<unsigned>(g), kThreads, 0, s>>>(
      static_cast<const uint16_t*>(a), P, static_cast<const uint16_t*>(b), Q, offsets, n_experts,
      cap_rows, c);
  return hipGetLastError();
}

}  // namespace moe
