// Grouped expert FFN in MXFP8 on gfx950's block-scaled matrix instructions
// (v_mfma_scale_f32_32x32x64_f8f6f4), fp32 accumulation.
//
// Page "Expert Parallel (EP)", Communication Pattern stage 3 and Requirements
// (tensor-style gate_up_proj / down_proj); page "Worked Example", Step 3; the
// MXFP8 transform named in torchtitan issue 5554. Format: OCP MX v1.0 MXFP8
// (E4M3 elements, one E8M0 scale per 32 values along K).
//
//   GEMM 1 (gated):  H[r, c] = bf16(SiLU(X[r,:] . Wgu[c,:]) * (X[r,:] . Wgu[I + c,:]))
//   GEMM 2:          Y[r, c] = H[r,:] . Wd[c,:]          (fp32)
// X and H are MXFP8 rows [M][K] with scales [M][K/32]; the weights are packed
// per output column, [N][K] with scales [N][K/32] (K contiguous), so both
// operands are staged and read the same way and no transposing LDS read is
// needed.
//
// Operand layout of the scaled 32x32x64 instruction (measured on the GPU):
// lane l holds 32 values of row (or column) l % 32; bytes 0..15 belong to the
// first 32-value K-block and bytes 16..31 to the second, and lane l's scale
// operand is the scale of row l % 32 in block l / 32. Within a block the two
// lane halves hold the two 16-value halves: lane half h takes K 16 h .. of
// each block, i.e. 16-byte chunks 4 kk + h and 4 kk + 2 + h of a 128-byte row
// for the slice kk (K 64 kk .. 64 kk + 63).
//
// Tiling (narrow tiles of the bf16 kernel): a workgroup of 4 waves computes up
// to 320 rows x 128 product columns; wave (wm, wn) owns up to 160 rows x 64
// (5 x 2 accumulator blocks). A K-step is 128 values (128 bytes per row, the
// bf16 kernel's row size), two MFMA slices. Activation and weight tiles are
// copied to LDS with the buffer-load-to-LDS path (1 KB per instruction,
// swizzled 16-byte chunks: chunk c of row r at c ^ (r & 7) ^ ((r >> 3) & 1));
// each row's 4 scale bytes of the step are copied as one dword per row.
// Activations run one step ahead (2 slots), weights two (3 slots). One
// workgroup per CU works through its share of the tile list.
#include <algorithm>
#include <cmath>

#include "moe_internal.h"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kThreads = 256;
constexpr int BM = 320;                 // rows per tile
constexpr int kMaxMB = 5;               // 32-row blocks per wave row
constexpr int WN = 64;                  // product columns per wave
constexpr int NQ = 2;                   // 32-column blocks per wave
constexpr int BNB = 2 * WN;             // product columns per tile (weight rows)
constexpr int BK = 128;                 // K per step (bytes per row)
constexpr int kTileA = BM * BK;         // 40 KB
constexpr int kTileB = BNB * BK;        // 16 KB
constexpr int NSB = 3;                  // weight ring slots
constexpr int NA = BM / 32;             // 1 KB activation copies per wave per step
constexpr int NB = BNB / 32;            // 1 KB weight copies per wave per step
constexpr int kSA = BM * 4;             // activation scale tile (one dword per row)
constexpr int kSB = BNB * 4;            // weight scale tile
constexpr int kXcds = 8;
constexpr int kMaxTableExperts = MOE_MAX_EXPERTS;
constexpr int kOutOfRange = 0x40000000;  // a load offset past every buffer (all < 2^30)

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int chunk_off(int row, int chunk) {
  return row * 128 + ((chunk ^ swz(row)) << 4);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes global -> LDS at lds_base + 16 * lane (M0 holds the LDS base).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff,
                                      unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_base) : "memory", "m0");
}
// 4 bytes global -> LDS at lds_base + 4 * lane, for the active lanes.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff,
                                     unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

enum Mode { kGateUp = 0, kDown = 1 };

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void ffn_gemm_mxfp8(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
    const int32_t* __restrict__ offsets, int n_experts, int64_t cap_rows,
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ Ws, void* __restrict__ Cout,
    int K, int N_out) {
  constexpr bool GATED = MODE == kGateUp;
  constexpr int BN_OUT = GATED ? BNB / 2 : BNB;
  constexpr int kLds = 2 * kTileA + NSB * kTileB + 2 * kSA + NSB * kSB;
  static_assert(kLds + 2 * (kMaxTableExperts + 1) * 4 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLds];
  __shared__ int s_tab[2 * (kMaxTableExperts + 1)];
  int* s_pref = s_tab;                         // tiles before expert e
  int* s_off = s_tab + kMaxTableExperts + 1;   // first row of expert e (clamped to cap)
  constexpr int kOffB = 2 * kTileA, kOffSA = kOffB + NSB * kTileB, kOffSB = kOffSA + 2 * kSA;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = (N_out + BN_OUT - 1) / BN_OUT;
  const int ncols = GATED ? 2 * N_out : N_out;  // packed weight rows per expert
  const int kb = K / 32;                        // scale bytes per row
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
  // Tiles of this workgroup: 8 contiguous runs of the tile list, run x served
  // by the workgroups b = x (mod 8) (XCD x), each taking every G8-th tile.
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
    const int n0 = nb * BN_OUT;

    // ---- copies (global -> LDS) ----
    // Activations: wave w copies 8-row groups NA w + i; lane -> row + (lane >> 3),
    // LDS chunk lane & 7 (global chunk swizzled). Rows past the segment read zeros.
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + static_cast<int64_t>(row_begin) * K), 0, rows * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t as_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(As + static_cast<int64_t>(row_begin) * kb), 0, rows * kb, 0x00020000);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + static_cast<int64_t>(expert) * ncols * K), 0, ncols * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t bs_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Ws + static_cast<int64_t>(expert) * ncols * kb), 0, ncols * kb, 0x00020000);
    int a_voff[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = 8 * (wave * NA + i) + (lane >> 3);
      a_voff[i] = row < rows ? row * K + (((lane & 7) ^ swz(row)) << 4) : kOutOfRange;
    }
    // Weight tile row j (0 .. BNB-1) = packed column: for GEMM 1 the first
    // half are gate columns n0 + j, the second the up columns N_out + n0 + ..;
    // columns past N_out read as zeros.
    auto wcol = [&](int j, bool& ok) {
      const int c = GATED ? n0 + (j % (BNB / 2)) : n0 + j;
      ok = c < N_out;
      return (GATED && j >= BNB / 2 ? N_out : 0) + c;
    };
    int b_voff[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = 8 * (wave * NB + i) + (lane >> 3);
      bool ok;
      const int c = wcol(j, ok);
      b_voff[i] = ok ? c * K + (((lane & 7) ^ swz(j)) << 4) : kOutOfRange;
    }
    // Scale dwords: wave w copies activation rows 80 w .. 80 w + 79 (two
    // instructions, 64 and 16 lanes) and weight rows 32 w .. 32 w + 31.
    const int sa_row0 = (BM / 4) * wave + lane, sa_row1 = sa_row0 + 64;
    const int sa_voff0 = sa_row0 < rows ? sa_row0 * kb : kOutOfRange;
    const int sa_voff1 = sa_row1 < rows ? sa_row1 * kb : kOutOfRange;
    int sb_voff;
    {
      bool ok;
      const int c = wcol((BNB / 4) * wave + lane, ok);
      sb_voff = ok ? c * kb : kOutOfRange;
    }
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_u8*)smem;

    // ---- compute assignment: wave (wm, wn) ----
    const int wm = wave >> 1, wn = wave & 1;
    const int nblk = (rows + 31) / 32;
    const int nmb = wm == 0 ? (nblk + 1) / 2 : nblk / 2;
    const int rowbase = wm == 0 ? 0 : 32 * ((nblk + 1) / 2);
    const int half = lane >> 5;
    // Fragment of slice kk: chunks 4 kk + half and 4 kk + 2 + half of the row.
    const int arow = rowbase + (lane & 31);
    int a_addr[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int p = 0; p < 2; ++p) a_addr[kk][p] = chunk_off(arow, 4 * kk + 2 * p + half);
    // Weight rows of column block q: GEMM 1 pairs gate block q with up block
    // q + NQ / 2 (same wave); GEMM 2 takes WN consecutive columns.
    int brow[NQ], b_addr[NQ][2][2];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      brow[q] = (GATED ? ((q < NQ / 2 ? 0 : BNB / 2) + wn * (WN / 2) + (q % (NQ / 2)) * 32)
                       : (wn * WN + q * 32)) + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int p = 0; p < 2; ++p) b_addr[q][kk][p] = chunk_off(brow[q], 4 * kk + 2 * p + half);
    }

    f32x16 acc[kMaxMB][NQ];
#pragma unroll
    for (int mb = 0; mb < kMaxMB; ++mb)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][q][r] = 0.f;

    // Copy item i of a step: activation copies 0..NA-1, the activation scale
    // copies NA, NA+1, then weight copies and the weight scale copy. All of a
    // step's activation-side items precede its weight-side items.
    constexpr int kItemsA = NA + 2, kItems = kItemsA + NB + 1;
    auto copy_item = [&](int i, bool do_a, int kt_a, int slot_a, bool do_b, int kt_b,
                         int slot_b) {
      if (i < NA) {
        if (do_a)
          dma16(a_rsrc, a_voff[i], kt_a * BK, lds0 + slot_a * kTileA + (wave * NA + i) * 1024);
      } else if (i == NA) {
        if (do_a) dma4(as_rsrc, sa_voff0, kt_a * 4, lds0 + kOffSA + slot_a * kSA + (BM / 4) * wave * 4);
      } else if (i == NA + 1) {
        if (do_a && lane < BM / 4 - 64)
          dma4(as_rsrc, sa_voff1, kt_a * 4,
               lds0 + kOffSA + slot_a * kSA + ((BM / 4) * wave + 64) * 4);
      } else if (i < kItemsA + NB) {
        if (do_b)
          dma16(b_rsrc, b_voff[i - kItemsA], kt_b * BK,
                lds0 + kOffB + slot_b * kTileB + (wave * NB + i - kItemsA) * 1024);
      } else if (i == kItemsA + NB) {
        if (do_b && lane < BNB / 4)
          dma4(bs_rsrc, sb_voff, kt_b * 4, lds0 + kOffSB + slot_b * kSB + (BNB / 4) * wave * 4);
      }
    };
    constexpr int kBItems = NB + 1;  // weight-side copies per step and wave

    auto run = [&](auto nmb_c) {
      constexpr int NMB = decltype(nmb_c)::value;
      // Prologue: weights of steps 0 and 1, activations of step 0.
#pragma unroll
      for (int i = kItemsA; i < kItems; ++i) copy_item(i, false, 0, 0, true, 0, 0);
#pragma unroll
      for (int i = 0; i < kItems; ++i) copy_item(i, true, 0, 0, nk > 1, 1, 1);
      int sb = 0;  // weight slot of step kt
      for (int kt = 0; kt < nk; ++kt) {
        const int sa = kt & 1;
        // This wave's copies of step kt are done (only the weight-side copies
        // of step kt + 1 may still be in flight); after the barrier every
        // wave's are, and every wave is done with step kt - 1's slots.
        if (kt + 1 < nk)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(kBItems));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
        const bool do_a = kt + 1 < nk, do_b = kt + 2 < nk;
        const int slot_a = sa ^ 1, slot_b = sb == 0 ? NSB - 1 : sb - 1;
        const unsigned char* abase = smem + sa * kTileA;
        const unsigned char* bbase = smem + kOffB + sb * kTileB;
        // Scales of the step: byte 2 kk + half of the row's dword is this
        // lane's block in slice kk (the instruction reads bits 0..7).
        unsigned sav[kMaxMB], sbv[NQ];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          sav[mb] = reinterpret_cast<const unsigned*>(smem + kOffSA + sa * kSA)[arow + mb * 32];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          sbv[q] = reinterpret_cast<const unsigned*>(smem + kOffSB + sb * kSB)[brow[q]];
        i32x8 fa[2][kMaxMB], fb[2][NQ];
        auto load = [&](int kk, i32x8(&xa)[kMaxMB], i32x8(&xb)[NQ]) {
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
            const uint4 lo = *reinterpret_cast<const uint4*>(abase + a_addr[kk][0] + mb * 32 * 128);
            const uint4 hi = *reinterpret_cast<const uint4*>(abase + a_addr[kk][1] + mb * 32 * 128);
            xa[mb] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                           (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          }
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const uint4 lo = *reinterpret_cast<const uint4*>(bbase + b_addr[q][kk][0]);
            const uint4 hi = *reinterpret_cast<const uint4*>(bbase + b_addr[q][kk][1]);
            xb[q] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          }
        };
        if (NMB > 0) load(0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (NMB > 0 && kk == 0) load(1, fa[1], fb[1]);
          __builtin_amdgcn_sched_barrier(0);
          const int sh = 16 * kk + 8 * half;
#pragma unroll
          for (int mb = 0; mb < kMaxMB; ++mb) {
            if (mb < NMB) {
#pragma unroll
              for (int q = 0; q < NQ; ++q)
                acc[mb][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fa[kk][mb], fb[kk][q], acc[mb][q], 0, 0, 0,
                    static_cast<int>(sav[mb] >> sh), 0, static_cast<int>(sbv[q] >> sh));
            }
            __builtin_amdgcn_sched_barrier(0);
            const int it = 2 * (kk * kMaxMB + mb);
            copy_item(it, do_a, kt + 1, slot_a, do_b, kt + 2, slot_b);
            copy_item(it + 1, do_a, kt + 1, slot_a, do_b, kt + 2, slot_b);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        sb = sb == NSB - 1 ? 0 : sb + 1;
      }
    };
    static_assert(kItems <= 2 * 2 * kMaxMB, "copy items fit the MFMA groups");
    switch (nmb) {
      case 5: run(std::integral_constant<int, 5>{}); break;
      case 4: run(std::integral_constant<int, 4>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      default: run(std::integral_constant<int, 0>{}); break;
    }
    if (nmb > 0) {
      // ---- epilogue ----
      // Accumulator register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4
      // and column l % 32 of its 32x32 block; a 4x4 transpose inside each group
      // of 4 lanes gives every lane 4 adjacent columns of one row.
      const int quad = lane & 3;
      auto transpose4 = [&](float (&v)[4]) {
        float nv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = __builtin_bit_cast(
              float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[r ^ 1]), 0xB1, 0xF, 0xF, false));
          nv[r] = ((r ^ quad) & 1) ? x : v[r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = __builtin_bit_cast(
              float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, nv[r ^ 2]), 0x4E, 0xF, 0xF, false));
          v[r] = ((r ^ quad) & 2) ? x : nv[r];
        }
      };
      const int row_end = row_begin + rows;
#pragma unroll
      for (int mb = 0; mb < kMaxMB; ++mb) {
        if (mb >= nmb) break;
#pragma unroll
        for (int q = 0; q < (GATED ? NQ / 2 : NQ); ++q) {
          const int col = n0 + (GATED ? wn * (WN / 2) : wn * WN) + q * 32 + (lane & 28);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * g + i;
              if (GATED) {
                const float gt = acc[mb][q][r], up = acc[mb][q + NQ / 2][r];
                v[i] = gt * up *
                       __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gt));
              } else {
                v[i] = acc[mb][q][r];
              }
            }
            transpose4(v);
            const int row = row_begin + rowbase + mb * 32 + 8 * g + 4 * half + quad;
            if (row < row_end && col < N_out) {
              const int64_t o = static_cast<int64_t>(row) * N_out + col;
              if (GATED)
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Cout) + o) = make_uint2(
                    f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16),
                    f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16));
              else
                *reinterpret_cast<float4*>(static_cast<float*>(Cout) + o) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
          }
        }
      }
    }
    // Every wave is done with this tile's LDS before the next tile's copies.
    __syncthreads();
  }
}

int num_cus_mx() {
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

// One workgroup per CU at most (rounded to the XCD count), one per tile bound
// below that.
template <int MODE>
hipError_t launch_ffn_mx(int n_experts, int64_t cap_rows, int K, int n_out, const void* a,
                         const void* as, const int32_t* offsets, const void* w, const void* ws,
                         void* out, hipStream_t s) {
  const int bn_out = MODE == kGateUp ? BNB / 2 : BNB;
  const int64_t mtiles = (cap_rows + BM - 1) / BM + (offsets ? n_experts : 0);
  const int64_t tiles = mtiles * ((n_out + bn_out - 1) / bn_out);
  const int64_t cus = std::max<int64_t>(kXcds, num_cus_mx() / kXcds * kXcds);
  const int64_t g = std::min((tiles + kXcds - 1) / kXcds * kXcds, cus);
  ffn_gemm_mxfp8<MODE><<<static_cast<unsigned>(g), kThreads, 0, s>>>(
      static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(as), offsets, n_experts,
      cap_rows, static_cast<const uint8_t*>(w), static_cast<const uint8_t*>(ws), out, K, n_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_mxfp8(int n_experts, int64_t cap_rows, int D, int inter,
                                const void* xq, const void* xs, const int32_t* offsets,
                                const void* wq, const void* wsc, void* h, hipStream_t s) {
  if (cap_rows == 0) return hipSuccess;
  return launch_ffn_mx<kGateUp>(n_experts, cap_rows, D, inter, xq, xs, offsets, wq, wsc, h, s);
}

hipError_t launch_down_mxfp8(int n_experts, int64_t cap_rows, int D, int inter, const void* hq,
                             const void* hs, const int32_t* offsets, const void* wq,
                             const void* wsc, void* y, hipStream_t s) {
  if (cap_rows == 0) return hipSuccess;
  return launch_ffn_mx<kDown>(n_experts, cap_rows, inter, D, hq, hs, offsets, wq, wsc, y, s);
}

}  // namespace moe
