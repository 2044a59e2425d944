// Grouped expert FFN for bf16 layers on gfx950 matrix cores (MFMA), fp32
// accumulation.
//
// Page "Expert Parallel (EP)", Communication Pattern stage 3 (each rank runs
// its local experts on the tokens it holds) and Requirements (tensor-style
// gate_up_proj / down_proj); page "Worked Example", Step 3 (a two-layer
// feed-forward network per expert).
//
//   GEMM 1 (gated):  H[r, c] = SiLU(X[r,:] . Wgu[:, c]) * (X[r,:] . Wgu[:, I + c])
//   GEMM 2:          Y[r, c] = H[r,:] . Wd[:, c]
// for the rows r of each expert's segment [offsets[e], offsets[e+1]).
//
// Precision: GEMM 1 multiplies the bf16 inputs exactly and accumulates in
// fp32. H is stored as fp16 (11 significant bits instead of bf16's 8: its
// rounding is the largest error of the layer, and fp16's range covers the
// gated activations), so GEMM 2 runs on the fp16 matrix instructions with
// each bf16 down_proj fragment converted to fp16 (round to nearest even) as
// it is read from LDS. Y is written in fp32 and rounded once, at the combine.
//
// Tiling. A 256-thread workgroup computes one tile of up to BM rows x 2 WN
// product columns over K in steps of 64; each wavefront owns up to BM / 2
// rows x WN products = (BM / 64) x (WN / 32) blocks of v_mfma_f32_32x32x16.
// Wide tiles: WN = 128, BM = 256 (256 accumulator registers, all of the
// AGPRs); narrow tiles: WN = 64, BM = 320 (160). Narrow tiles are used when
// wide ones would leave CUs idle. For GEMM 1 the product columns are gate columns and the matching up
// columns, each wave holding both halves, so the SiLU-gate epilogue pairs
// them in registers.
//
// Staging. Global -> LDS copies use the buffer-load-to-LDS path (no register
// round trip), 1 KB per instruction. Activation tiles run one K-step ahead (a
// ring of 2); weight tiles two steps ahead (a ring of 3) when that fits in
// LDS, else one (WN = 128: a ring of 2); a step's copies are spread between
// its MFMA groups so the wave keeps the matrix core busy while they issue. LDS layouts (conflict-free reads):
//  * activations, [row][64] x 16-bit (128-byte rows); 16-byte chunk c of row
//    r sits at chunk c ^ (r & 7) ^ ((r >> 3) & 1). A fragment is one 16-byte
//    read per lane.
//  * weights, [k][2 WN] x 16-bit (N contiguous as in memory); 16-byte chunk c
//    of row k sits at chunk c ^ 4 (k & 3). A fragment (8 K-values of
//    one column per lane) is two ds_read_b64_tr_b16 transposing reads.
// The swizzles are applied to the global addresses of the copies, so each
// copy instruction writes 1 KB of LDS linearly.
//
// Ragged experts. Tiles are listed in the order (expert, column block, row
// block) from the device-resident offsets, so the grid is sized from the row
// capacity and needs no host synchronisation; surplus workgroups exit at
// once. An expert's rows are cut into near-equal row blocks of at most BM
// rows (narrow tiles: segments of 460..640 rows make two blocks, not three);
// the 32-row slices holding rows are shared out between the two wave rows, and
// a wave skips the MFMAs (and fragment reads) of slices past the segment. The tile list is dealt to the 8 XCDs in contiguous runs
// (workgroup b runs on XCD b mod 8), so the row blocks that share a weight
// tile, and the column blocks that share an activation tile, meet in one
// XCD's L2.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kThreads = 256;
constexpr int BK = 64;                 // K per step
// Rows per tile for WN product columns per wave.
constexpr int bm_of(int wn) { return wn == 128 ? 256 : 320; }
constexpr int kXcds = 8;
constexpr int kMaxTableExperts = MOE_MAX_EXPERTS;
constexpr int kOutOfRange = 0x40000000;  // a load offset past every buffer (all < 2^30)

__device__ __forceinline__ int a_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int a_off(int row, int chunk) {
  return row * 128 + ((chunk ^ a_swz(row)) << 4);
}
// Weight tile rows are ROWB = 2 * BNB bytes.
template <int ROWB>
__device__ __forceinline__ int b_off(int k, int col) {
  return k * ROWB + (((col >> 3) ^ ((k & 3) << 2)) << 4) + ((col & 7) << 1);
}

__device__ __forceinline__ uint32_t f16_bits(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<_Float16>(f));  // round to nearest even
}

// Two bf16 values -> two fp16 values (round to nearest even): widen both to
// fp32 exactly, then one packed conversion (v_cvt_pk_f16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  const f32x2 f = {__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// 16 bytes global -> LDS at lds_base + 16 * lane: buffer_load_dwordx4 with the
// LDS destination (M0 holds the LDS base). Out-of-range offsets write zeros.
// The loads are counted by vmcnt; the caller waits before reading the LDS.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff,
                                      unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate that waits until at most n (< 64) vector memory
// operations of this wave are outstanding (lgkm and exp counters unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// GEMM 1: bf16 x bf16 -> SiLU(gate) * up -> fp16 H.
// GEMM 2: fp16 H x (bf16 -> fp16) W_down -> fp32 Y.
// GEMM 1 in the backward pass (the pre-activations G, U are recomputed and
// kept in the accumulators): with dH [rows, N_out] fp32 read in the
// epilogue, writes dG | dU = dH U SiLU'(G) | dH SiLU(G) ([rows, 2 N_out],
// bf16) and H = SiLU(G) U ([rows, N_out], bf16).
// GEMM 1 of a training forward: as kGateUp, and the pre-activations G | U
// are also stored in fp32 ([rows, 2 N_out], gu_out) for the backward.
enum Mode { kGateUp = 0, kDown = 1, kGateUpBwd = 2, kGateUpSave = 3 };

// WN: product columns per wave (128 or 64); a tile has BNB = 2 WN product
// columns.
template <int MODE, int WN>
__global__ __launch_bounds__(kThreads, 1) void ffn_gemm_bf16(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int n_experts,
    int64_t cap_rows, const uint16_t* __restrict__ W, void* __restrict__ Cout, int K,
    int N_out, const float* __restrict__ dh_in, uint16_t* __restrict__ h_out,
    const uint16_t* const* __restrict__ w_ptrs, float* __restrict__ gu_out) {
  constexpr bool GATED = MODE != kDown;  // gate and up columns paired in a wave
  constexpr int BM = bm_of(WN);
  constexpr int kMaxMB = BM / 64;        // 32-row blocks per wave row
  constexpr int kTileA = BM * BK * 2;
  constexpr int NA = BM / 32;            // 1 KB activation copies per wave per step
  constexpr int BNB = 2 * WN;
  constexpr int NQ = WN / 32;                 // 32-column blocks per wave
  constexpr int ROWB = 2 * BNB;               // bytes per weight row in LDS
  constexpr int kTileB = BK * ROWB;
  constexpr int BN_OUT = GATED ? BNB / 2 : BNB;
  // Narrow tiles: one workgroup per CU works through several tiles, so the
  // tile table has LDS of its own. Wide tiles: one tile per workgroup, the
  // table lives in the staging memory until the first copy (a separate table
  // would cost the weight ring its third slot).
  constexpr bool kPersist = WN == 64;
  // LDS: activation ring of 2 tiles, then a weight ring of NSB tiles (and the
  // tile table).
  constexpr int kTabInts = 2 * (kMaxTableExperts + 1);
  constexpr int kTab = kPersist ? kTabInts * 4 : 0;
  constexpr int NSB = 2 * kTileA + 3 * kTileB + kTab <= 160 * 1024 ? 3 : 2;
  constexpr int kLds = 2 * kTileA + NSB * kTileB;
  static_assert(kLds + kTab <= 160 * 1024, "LDS budget");
  static_assert(kTabInts * 4 <= kLds, "the table fits in the staging memory");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLds];
  __shared__ int s_tab[kPersist ? kTabInts : 1];
  int* s_pref = kPersist ? s_tab : reinterpret_cast<int*>(smem);  // tiles before expert e
  int* s_off = s_pref + kMaxTableExperts + 1;  // first row of expert e (clamped to cap)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int NT = (N_out + BN_OUT - 1) / BN_OUT;
  const int ldw = GATED ? 2 * N_out : N_out;
  const int nk = K / BK;
  const int n_exp = offsets ? n_experts : 1;

  // ---- tile table: per-expert prefix of tile counts ----
  if (wave == 0) {
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
  // Tiles of this workgroup: the tile list [0, R) is cut into 8 contiguous
  // runs of ceil(R / 8), run x served by the workgroups b = x (mod 8) (the
  // workgroups of XCD x); workgroup b takes tiles x * per + b / 8 + i * G8 of
  // the run, G8 = its XCD's workgroup count. One tile each when the grid
  // covers the tile list; several, one after another, when the grid is one
  // workgroup per CU.
  const int G8 = static_cast<int>(gridDim.x) / kXcds;
  const int xcd = static_cast<int>(blockIdx.x) % kXcds, slot = static_cast<int>(blockIdx.x) / kXcds;
  const int per = (R + kXcds - 1) / kXcds;
  const int run_end = min((xcd + 1) * per, R);
  for (int t = xcd * per + slot; t < run_end; t += G8) {
    // The lane index passes through an empty asm statement, so values derived
    // from it are computed per tile instead of being hoisted out of the tile
    // loop (where they would outlive the accumulators' registers and spill).
    int lane_t = tid & 63;
    asm volatile("" : "+v"(lane_t));
    const int lane = lane_t;

    // Tile t -> expert (the number of experts whose tiles end at or before t),
    // column block and row block. Wave-uniform.
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
    // The segment's rows are cut into mt near-equal row blocks of at most BM.
    const int cnt = seg_end - seg_beg;
    const int mt = (cnt + BM - 1) / BM;
    const int chunk = (cnt + mt - 1) / mt;
    const int nb = local / mt, mbk = local - nb * mt;
    const int row_begin = seg_beg + mbk * chunk;
    const int rows = min(chunk, seg_end - row_begin);  // <= BM
    if (rows <= 0) continue;  // (uniform: the whole workgroup takes the same tile)
    const int n0 = nb * BN_OUT;
    if (!kPersist) __syncthreads();  // every wave has read the table

    // ---- copy assignment (global -> LDS), fixed for the tile ----
    // Activations: wave w copies the 8-row groups g = NA w + i (i < NA), rows
    // 8g .. 8g + 7; lane -> row 8g + (lane >> 3), LDS chunk lane & 7 (global
    // chunk swizzled). Rows past the segment lie past the buffer's end and read
    // as zeros. (Skipping whole groups past the segment instead makes the
    // compiler unswitch the K loop on that test, duplicating it with
    // accumulator copies.)
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + static_cast<int64_t>(row_begin) * K), 0, rows * K * 2, 0x00020000);
    // Stacked experts ([n, K, ldw]) or one buffer per expert (w_ptrs[expert]).
    const uint16_t* wexp = w_ptrs ? w_ptrs[expert] : W + static_cast<int64_t>(expert) * K * ldw;
    const __amdgpu_buffer_rsrc_t b_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)wexp, 0, K * ldw * 2, 0x00020000);
    int a_voff[NA];
  #pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = 8 * (wave * NA + i) + (lane >> 3);
      a_voff[i] = row < rows ? row * K * 2 + (((lane & 7) ^ a_swz(row)) << 4) : kOutOfRange;
    }
    // Weights: the tile has 64 rows of ROWB bytes; wave w copies KB = ROWB / 64
    // rows per instruction, NB = kTileB / 4 KB instructions. Lane -> LDS chunk
    // lane % CH of its row (CH = ROWB / 16 chunks). For GEMM 1 the first half of
    // the chunks are gate columns n0.., the second half the up columns I + n0..;
    // columns past N_out read as zeros.
    constexpr int CH = ROWB / 16;
    constexpr int KB = 64 / CH;
    constexpr int NB = kTileB / 4096;
    int b_voff[NB];
  #pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int k = KB * (wave * NB + i) + lane / CH;
      const int gch = (lane % CH) ^ ((k & 3) << 2);
      const int c = GATED ? (gch % (CH / 2)) * 8 : gch * 8;
      const int col = (GATED && gch >= CH / 2 ? N_out : 0) + n0 + c;
      b_voff[i] = n0 + c < N_out ? (k * ldw + col) * 2 : kOutOfRange;
    }
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_u8*)smem;

    // ---- compute assignment: wave (wm, wn) ----
    // The tile's 32-row blocks holding rows of the segment are shared out
    // between the two wave rows (wm = 0 takes the first ceil(n/2)), so a
    // partial tile keeps both wave rows busy. Wave wn owns product columns
    // wn * WN .. (for GEMM 1: gate columns wn * WN/2 .. and the same up columns).
    const int wm = wave >> 1, wn = wave & 1;
    const int nblk = (rows + 31) / 32;
    const int nmb = wm == 0 ? (nblk + 1) / 2 : nblk / 2;
    const int rowbase = wm == 0 ? 0 : 32 * ((nblk + 1) / 2);
    const int half = lane >> 5;
    const int grp = lane >> 4, j16 = lane & 15;
    // A fragment of row block mb, K-slice kk: row rowbase + mb*32 + lane%32,
    // chunk 2 kk + half (the swizzle does not depend on rowbase or mb).
    int a_addr[4];
  #pragma unroll
    for (int kk = 0; kk < 4; ++kk) a_addr[kk] = a_off(rowbase + (lane & 31), kk * 2 + half);
    // B fragment of column block q: lane j of 16-lane group g reads 8 bytes of
    // weight row 8 (g >> 1) + (j >> 2) (+4 for the second read) at column
    // blk + 16 (g & 1) + 4 (j & 3); lane l then holds K-values 8 (l >> 5) ..
    // + 7 of column blk + l % 32.
    int b_addr[NQ];
  #pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int blk = GATED ? ((q < NQ / 2 ? 0 : BNB / 2) + wn * (WN / 2) + (q % (NQ / 2)) * 32)
                            : (wn * WN + q * 32);
      b_addr[q] = b_off<ROWB>(8 * (grp >> 1) + (j16 >> 2), blk + 16 * (grp & 1) + 4 * (j16 & 3));
    }

    f32x16 acc[kMaxMB][NQ];
  #pragma unroll
    for (int mb = 0; mb < kMaxMB; ++mb)
  #pragma unroll
      for (int q = 0; q < NQ; ++q)
  #pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][q][r] = 0.f;

    auto run = [&](auto nmb_c) {
      constexpr int NMB = decltype(nmb_c)::value;
      auto load_frags = [&](int sa, int sb, int kk, uint4(&fa)[kMaxMB], uint4(&fb)[NQ]) {
        const unsigned char* abase = smem + sa * kTileA;
  #pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          fa[mb] = *reinterpret_cast<const uint4*>(abase + a_addr[kk] + mb * 32 * 128);
        const lds_u8* bbase = (const lds_u8*)smem + 2 * kTileA + sb * kTileB;
  #pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const lds_u8* p = bbase + b_addr[q] + kk * 16 * ROWB;
          const uint2 lo =
              __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
          const uint2 hi = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * ROWB)));
          fb[q] = make_uint4(lo.x, lo.y, hi.x, hi.y);
          if (MODE == kDown) {
            fb[q].x = bf16x2_to_f16x2(fb[q].x);
            fb[q].y = bf16x2_to_f16x2(fb[q].y);
            fb[q].z = bf16x2_to_f16x2(fb[q].z);
            fb[q].w = bf16x2_to_f16x2(fb[q].w);
          }
        }
      };
      // MFMAs of row block mb for one K-slice.
      auto mfma_row = [&](int mb, const uint4(&fa)[kMaxMB], const uint4(&fb)[NQ]) {
  #pragma unroll
        for (int q = 0; q < NQ; ++q) {
          if (MODE != kDown)
            acc[mb][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, fa[mb]), __builtin_bit_cast(bf16x8, fb[q]), acc[mb][q],
                0, 0, 0);
          else
            acc[mb][q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, fa[mb]), __builtin_bit_cast(f16x8, fb[q]), acc[mb][q],
                0, 0, 0);
        }
      };
      // Copy item i of a step: activation copies 0..NA-1 first, then weight
      // copies NA..NA+NB-1. A step's items are spread over its 4 kMaxMB MFMA
      // groups so that the wave keeps the matrix core busy while the copies
      // issue.
      auto copy_item = [&](int i, bool do_a, int kt_a, int slot_a, bool do_b, int kt_b,
                           int slot_b) {
        if (i < NA) {
          if (do_a)
            dma16(a_rsrc, a_voff[i], kt_a * BK * 2,
                  lds0 + slot_a * kTileA + (wave * NA + i) * 1024);
        } else if (i - NA < NB) {
          if (do_b)
            dma16(b_rsrc, b_voff[i - NA], kt_b * BK * ldw * 2,
                  lds0 + 2 * kTileA + slot_b * kTileB + (wave * NB + i - NA) * 1024);
        }
      };
      // Activations run one step ahead (2 slots), weights NSB - 1 steps ahead.
      // Copies complete in issue order; within a step all activation copies
      // precede the weight copies, so with a 3-slot weight ring, when this
      // wave's copies for A(k) are done, at most the NB weight copies of step
      // k + 1 are still in flight; with a 2-slot ring, all of step k's copies
      // are waited for.
      if (NSB == 3) {
  #pragma unroll
        for (int i = NA; i < NA + NB; ++i) copy_item(i, false, 0, 0, true, 0, 0);
      }
  #pragma unroll
      for (int i = 0; i < NA + NB; ++i)
        copy_item(i, true, 0, 0, NSB == 2 || nk > 1, NSB - 2, NSB - 2);
      int sb = 0;  // weight slot of step kt
      for (int kt = 0; kt < nk; ++kt) {
        const int sa = kt & 1;
        // This wave's copies of step kt are done; after the barrier every
        // wave's are, and every wave has finished step kt - 1, whose slots the
        // next copies overwrite.
        if (NSB == 3 && kt + 1 < nk)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(NB));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
        const bool do_a = kt + 1 < nk, do_b = kt + NSB - 1 < nk;
        const int slot_a = sa ^ 1, slot_b = sb == 0 ? NSB - 1 : sb - 1;
        // The fragments of K-slice kk + 1 are read while slice kk multiplies;
        // the scheduling barriers fix this order (the compiler would otherwise
        // sink the reads next to their first use).
        uint4 fa[2][kMaxMB], fb[2][NQ];
        if (NMB > 0) load_frags(sa, sb, 0, fa[0], fb[0]);
  #pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (NMB > 0 && kk < 3) load_frags(sa, sb, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int mb = 0; mb < kMaxMB; ++mb) {
            if (mb < NMB) mfma_row(mb, fa[kk & 1], fb[kk & 1]);
            __builtin_amdgcn_sched_barrier(0);
            copy_item(kk * kMaxMB + mb, do_a, kt + 1, slot_a, do_b, kt + NSB - 1, slot_b);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        sb = sb == NSB - 1 ? 0 : sb + 1;
      }
    };
    // kGateUpBwd: the epilogue's dH values of row block 0 are loaded before
    // the K loop (issued ahead of its copies, so the copies' vmcnt waits also
    // cover them); those of row block mb + 1 while block mb is computed.
    constexpr int NQD = MODE == kGateUpBwd ? NQ / 2 : 1;
    float4 dpre[2][NQD][4];
    auto load_dh = [&](int mb, float4(&d)[NQD][4]) {
  #pragma unroll
      for (int q = 0; q < NQD; ++q) {
        const int col = n0 + wn * (WN / 2) + q * 32 + (lane & 28);
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = row_begin + rowbase + mb * 32 + 8 * g + 4 * half + (lane & 3);
          d[q][g] = row < row_begin + rows && col < N_out
                        ? *reinterpret_cast<const float4*>(dh_in + static_cast<int64_t>(row) * N_out + col)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    };
    if (MODE == kGateUpBwd && nmb > 0) load_dh(0, dpre[0]);
    static_assert(kMaxMB <= 5 && NA + NB <= 4 * kMaxMB, "copy items fit the MFMA groups");
    switch (nmb) {
      case 5:  // narrow tiles only (rows <= 256 give nmb <= 4)
        if constexpr (kMaxMB == 5) run(std::integral_constant<int, 5>{});
        break;
      case 4: run(std::integral_constant<int, 4>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      default: run(std::integral_constant<int, 0>{}); break;
    }
    if (nmb > 0) {
      // ---- epilogue ----
      // Accumulator register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4
      // and column l % 32 of its 32x32 block. A 4x4 transpose inside each group of
      // 4 lanes (two DPP exchange rounds) gives every lane 4 adjacent columns of
      // one row, so each store writes 8 (fp16) or 16 (fp32) bytes.
      const int quad = lane & 3;
      auto transpose4 = [&](float (&v)[4]) {
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
      };
      const int row_end = row_begin + rows;
    #pragma unroll
      for (int mb = 0; mb < kMaxMB; ++mb) {
        if (mb >= nmb) break;
        if (MODE == kGateUpBwd && mb + 1 < nmb) load_dh(mb + 1, dpre[(mb + 1) & 1]);
    #pragma unroll
        for (int q = 0; q < (GATED ? NQ / 2 : NQ); ++q) {
          const int col = n0 + (GATED ? wn * (WN / 2) : wn * WN) + q * 32 + (lane & 28);
    #pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int row = row_begin + rowbase + mb * 32 + 8 * g + 4 * half + quad;
            if (MODE == kGateUpBwd) {
              float gv[4], uv[4];
    #pragma unroll
              for (int i = 0; i < 4; ++i) {
                gv[i] = acc[mb][q][4 * g + i];
                uv[i] = acc[mb][q + NQ / 2][4 * g + i];
              }
              transpose4(gv);
              transpose4(uv);
              if (row < row_end && col < N_out) {
                const int64_t o = static_cast<int64_t>(row) * N_out + col;
                const float4 d4 = dpre[mb & 1][q < NQD ? q : 0][g];
                const float dh[4] = {d4.x, d4.y, d4.z, d4.w};
                uint32_t dgw[2], duw[2], hw[2];
    #pragma unroll
                for (int i = 0; i < 4; i += 2) {
                  float dg[2], du[2], hv[2];
    #pragma unroll
                  for (int e = 0; e < 2; ++e) {
                    // s = sigmoid(g), SiLU(g) = g s, SiLU'(g) = s + SiLU(g) (1 - s)
                    const float gt = gv[i + e], up = uv[i + e];
                    const float sg = __builtin_amdgcn_rcpf(
                        1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gt));
                    const float silu = gt * sg;
                    dg[e] = dh[i + e] * up * (sg + silu * (1.f - sg));
                    du[e] = dh[i + e] * silu;
                    hv[e] = silu * up;
                  }
                  dgw[i / 2] = f32_to_bf16(dg[0]) | (static_cast<uint32_t>(f32_to_bf16(dg[1])) << 16);
                  duw[i / 2] = f32_to_bf16(du[0]) | (static_cast<uint32_t>(f32_to_bf16(du[1])) << 16);
                  hw[i / 2] = f32_to_bf16(hv[0]) | (static_cast<uint32_t>(f32_to_bf16(hv[1])) << 16);
                }
                uint16_t* dgu = static_cast<uint16_t*>(Cout) + static_cast<int64_t>(row) * 2 * N_out + col;
                *reinterpret_cast<uint2*>(dgu) = make_uint2(dgw[0], dgw[1]);
                *reinterpret_cast<uint2*>(dgu + N_out) = make_uint2(duw[0], duw[1]);
                *reinterpret_cast<uint2*>(h_out + o) = make_uint2(hw[0], hw[1]);
              }
              continue;
            }
            if (MODE == kGateUp || MODE == kGateUpSave) {
              // G and U moved to row-major lanes first, then H = SiLU(G) U:
              // one code path for both forward modes, so the training
              // forward's H (and y) is the plain forward's, bit for bit.
              float gv[4], uv[4];
    #pragma unroll
              for (int i = 0; i < 4; ++i) {
                gv[i] = acc[mb][q][4 * g + i];
                uv[i] = acc[mb][q + NQ / 2][4 * g + i];
              }
              transpose4(gv);
              transpose4(uv);
              if (row < row_end && col < N_out) {
                if (MODE == kGateUpSave) {
                  float* o = gu_out + static_cast<int64_t>(row) * 2 * N_out + col;
                  *reinterpret_cast<float4*>(o) = make_float4(gv[0], gv[1], gv[2], gv[3]);
                  *reinterpret_cast<float4*>(o + N_out) = make_float4(uv[0], uv[1], uv[2], uv[3]);
                }
                float v[4];
    #pragma unroll
                for (int i = 0; i < 4; ++i)
                  // SiLU(g) u = g u / (1 + exp(-g)), exp via exp2, then reciprocal
                  v[i] = gv[i] * uv[i] *
                         __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gv[i]));
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Cout) +
                                          static_cast<int64_t>(row) * N_out + col) =
                    make_uint2(f16_bits(v[0]) | (f16_bits(v[1]) << 16),
                               f16_bits(v[2]) | (f16_bits(v[3]) << 16));
              }
              continue;
            }
            // kDown: fp32 Y.
            float v[4];
    #pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[mb][q][4 * g + i];
            transpose4(v);
            if (row < row_end && col < N_out)
              *reinterpret_cast<float4*>(static_cast<float*>(Cout) +
                                         static_cast<int64_t>(row) * N_out + col) =
                  make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
    // Every wave is done with this tile's LDS before the next tile's copies.
    __syncthreads();
  }
}

// Workgroups to launch: an upper bound of the tile count (each expert's
// segment may end in a partial row block: at most one extra per expert),
// rounded up to a multiple of the XCD count.
int64_t tile_bound(int64_t cap_rows, const int32_t* offsets, int n_experts, int n_out,
                   int bn_out, int BM) {
  const int64_t mtiles = (cap_rows + BM - 1) / BM + (offsets ? n_experts : 0);
  return mtiles * ((n_out + bn_out - 1) / bn_out);
}
int num_cus();

// Workgroups to launch for at most `tiles` tiles: one per tile, rounded up to
// a multiple of the XCD count. With `persist` at most one per CU, each then
// working through its share of the tile list (the tile table is built once
// per workgroup and no workgroup is launched per tile).
unsigned grid_of(int64_t tiles, bool persist) {
  const int64_t g = (tiles + kXcds - 1) / kXcds * kXcds;
  if (!persist) return static_cast<unsigned>(g);
  const int64_t cus = std::max<int64_t>(kXcds, num_cus() / kXcds * kXcds);
  return static_cast<unsigned>(std::min(g, cus));
}

int num_cus() {
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

// Wide tiles (128 columns per wave) unless narrow ones (64) are expected to
// finish sooner. The estimate counts waves of tiles over the CUs. Row blocks:
// each expert's share of cap_rows, spread as routing noise spreads it (the
// counts at mean -1.5, -0.5, +0.5 and +1.5 standard deviations, sqrt(mean)),
// cut into blocks of at most BM rows. A narrow tile (320 x 128 products)
// costs about 2/3 of a wide one (256 x 256; measured on the grouped GEMMs).
template <int MODE>
hipError_t launch_ffn(int n_experts, int64_t cap_rows, int K, int n_out, const void* a,
                      const int32_t* offsets, const void* w, void* out, hipStream_t s,
                      const float* dh_in = nullptr, void* h_out = nullptr,
                      const void* const* w_ptrs = nullptr, float* gu_out = nullptr) {
  constexpr int kWideOut = MODE != kDown ? 128 : 256;
  const int64_t ne = offsets ? n_experts : 1;
  const double mean = static_cast<double>(cap_rows) / static_cast<double>(ne);
  const double sd = offsets ? std::sqrt(mean) : 0.0;
  const int64_t cus = num_cus();
  auto waves = [&](int bm, int bn_out) {
    int64_t q4 = 0;  // 4 x the expected row blocks of one expert
    for (const double z : {-1.5, -0.5, 0.5, 1.5}) {
      const int64_t rows = static_cast<int64_t>(std::ceil(std::max(mean + z * sd, 1.0)));
      q4 += (rows + bm - 1) / bm;
    }
    const int64_t tiles = (ne * q4 + 3) / 4 * ((n_out + bn_out - 1) / bn_out);
    return (tiles + cus - 1) / cus;
  };
  const int64_t waves_w = waves(bm_of(128), kWideOut);
  const int64_t waves_n = waves(bm_of(64), kWideOut / 2);
  const bool wide = 3 * waves_w <= 2 * waves_n;
  if (wide) {
    const unsigned g =
        grid_of(tile_bound(cap_rows, offsets, n_experts, n_out, kWideOut, bm_of(128)), false);
    ffn_gemm_bf16<MODE, 128><<<g, kThreads, 0, s>>>(static_cast<const uint16_t*>(a), offsets,
                                                    n_experts, cap_rows,
                                                    static_cast<const uint16_t*>(w), out, K, n_out,
                                                    dh_in, static_cast<uint16_t*>(h_out),
                                                    reinterpret_cast<const uint16_t* const*>(w_ptrs),
                                                    gu_out);
  } else {
    const unsigned g =
        grid_of(tile_bound(cap_rows, offsets, n_experts, n_out, kWideOut / 2, bm_of(64)), true);
    ffn_gemm_bf16<MODE, 64><<<g, kThreads, 0, s>>>(static_cast<const uint16_t*>(a), offsets,
                                                   n_experts, cap_rows,
                                                   static_cast<const uint16_t*>(w), out, K, n_out,
                                                   dh_in, static_cast<uint16_t*>(h_out),
                                                   reinterpret_cast<const uint16_t* const*>(w_ptrs),
                                                   gu_out);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_bf16(int n_experts, int64_t cap_rows, int D, int inter,
                               const void* x_perm, const int32_t* offsets, const void* w_gate_up,
                               void* h, hipStream_t s, const void* const* w_ptrs) {
  if (cap_rows == 0) return hipSuccess;
  return launch_ffn<kGateUp>(n_experts, cap_rows, D, inter, x_perm, offsets, w_gate_up, h, s,
                             nullptr, nullptr, w_ptrs);
}

hipError_t launch_gate_up_save_bf16(int n_experts, int64_t cap_rows, int D, int inter,
                                    const void* x_perm, const int32_t* offsets,
                                    const void* w_gate_up, void* h, float* gu, hipStream_t s) {
  if (cap_rows == 0) return hipSuccess;
  return launch_ffn<kGateUpSave>(n_experts, cap_rows, D, inter, x_perm, offsets, w_gate_up, h, s,
                                 nullptr, nullptr, nullptr, gu);
}

hipError_t launch_gate_up_bwd_bf16(int n_experts, int64_t cap_rows, int D, int inter,
                                   const void* x_perm, const int32_t* offsets,
                                   const void* w_gate_up, const float* dh, void* dgu, void* h,
                                   hipStream_t s) {
  if (cap_rows == 0) return hipSuccess;
  return launch_ffn<kGateUpBwd>(n_experts, cap_rows, D, inter, x_perm, offsets, w_gate_up, dgu,
                                s, dh, h);
}

hipError_t launch_down_bf16(int n_experts, int64_t cap_rows, int D, int inter, const void* h,
                            const int32_t* offsets, const void* w_down, void* y, hipStream_t s,
                            const void* const* w_ptrs) {
  if (cap_rows == 0) return hipSuccess;
  return launch_ffn<kDown>(n_experts, cap_rows, inter, D, h, offsets, w_down, y, s, nullptr,
                           nullptr, w_ptrs);
}

}  // namespace moe
