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
// gated activations; a value beyond +-65504 saturates there instead of
// becoming infinite), so GEMM 2 runs on the fp16 matrix instructions with
// each bf16 down_proj fragment converted to fp16 (round to nearest even) as
// it is read from LDS. Y is written in fp32 and rounded once, at the combine.
//
// Tiling. A 256-thread workgroup computes one tile of up to BM rows x 2 WN
// product columns over K in steps of 64; in the 2 x 2 wave layout each
// wavefront owns up to BM / 2 rows x WN products = (BM / 64) x (WN / 32)
// blocks of v_mfma_f32_32x32x16. Wide tiles: WN = 128, BM = 256 (256
// accumulator registers, all of the AGPRs); narrow tiles: WN = 64, BM = 320
// (160). Narrow tiles are used when wide ones would leave CUs idle. The down
// GEMM's wide packed tiles use a 1 x 4 layout instead (each wave all 256 rows
// x 64 columns, the same 256 accumulators). For GEMM 1 the product columns
// are gate columns and the matching up columns, each wave holding both
// halves, so the SiLU-gate epilogue pairs them in registers.
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
// Packed weights (the operand order launch_pack_weights writes: per
// 32-column block and 16-deep K slice, 1 KB with each lane's 16 bytes
// contiguous; down_proj already in fp16). Each wave loads its own weight
// fragments straight into registers, one 16-byte load per lane and fragment,
// and only the activations go through LDS (two slots, one step ahead). A
// step's slice-kk fragments of the next step are loaded as soon as this
// step's slice-kk MFMAs have read them. This halves the kernel's LDS traffic
// (no weight copies into LDS, no weight reads from it) for twice the weight
// reads from L2 (both wave rows load the same fragments).
//
// Ragged experts. Tiles are listed in the order (expert, row-block group,
// column block, row block) from the device-resident offsets, so the grid is sized from the row
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
// Split-K tail: at most kMaxSplit parts of at least kMinSplitSteps K-steps
// (shorter parts do not pay for writing and re-reading their accumulators
// and lose the tile order's L2 sharing: measured on the rank-share layer,
// K = 2048 in 3 parts, the down GEMM took 1087 us against 1055 us whole,
// while the Mixtral-style one, K = 14336 in 5 parts, went 1837 -> 1649 us).
constexpr int kMaxSplit = 8;
constexpr int kMinSplitSteps = 32;
// The gated GEMM's parts may be shorter (its K, the model width, is short next
// to the down GEMM's): measured with 16, the Mixtral-style gate_up GEMM
// (K = 64 steps, 3 parts) went 3170 -> 3150 us, the skewed layer's (32 steps,
// 2 parts of 16) 785 -> 803 us; 20 keeps the first and leaves the second
// whole.
constexpr int kMinSplitStepsGated = 20;
template <int MODE>
constexpr int min_split_steps() { return MODE == 1 ? kMinSplitSteps : kMinSplitStepsGated; }

__device__ __forceinline__ int a_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int a_off(int row, int chunk) {
  return row * 128 + ((chunk ^ a_swz(row)) << 4);
}
// Weight tile rows are ROWB = 2 * BNB bytes.
template <int ROWB>
__device__ __forceinline__ int b_off(int k, int col) {
  return k * ROWB + (((col >> 3) ^ ((k & 3) << 2)) << 4) + ((col & 7) << 1);
}

// fp32 -> fp16 bits, round to nearest even, saturating at +-65504 (fp16's
// largest finite value) so that a finite H never becomes infinite; NaN stays
// NaN (both comparisons are false).
__device__ __forceinline__ uint32_t f16_sat_bits(float f) {
  const float c = f > 65504.f ? 65504.f : (f < -65504.f ? -65504.f : f);
  return __builtin_bit_cast(unsigned short, static_cast<_Float16>(c));
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
// The same, and no LDS (or scalar memory) operation of this wave outstanding.
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// GEMM 1: bf16 x bf16 -> SiLU(gate) * up -> fp16 H.
// GEMM 2: fp16 H x (bf16 -> fp16) W_down -> fp32 Y.
// GEMM 1 in the backward pass (the pre-activations G, U are recomputed and
// kept in the accumulators): with dH [rows, N_out] fp32 read in the
// epilogue, writes dG | dU = dH U SiLU'(G) | dH SiLU(G) ([rows, 2 N_out],
// bf16) and H = SiLU(G) U ([rows, N_out], bf16).
// GEMM 1 of a training forward: as kGateUp, and the pre-activations G | U
// are also stored in fp32 ([rows, 2 N_out], gu_out) for the backward.
enum Mode { kGateUp = 0, kDown = 1, kGateUpBwd = 2, kGateUpSave = 3 };

// One 32x32x16 product added into c (activation fragment xa, weight fragment
// wb). Gated GEMMs give the weight fragment as the MFMA's first operand, so
// the block comes out transposed: register r of lane l holds output column
// 8 (r / 4) + 4 (l / 32) + r % 4 and row l % 32, i.e. every lane holds runs of
// 4 adjacent columns of one row, which the epilogue stores as they are. The
// down GEMM keeps the plain order (register r of lane l: row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32) and its epilogue exchanges
// values inside groups of 4 lanes: with the transposed order its epilogue
// ran out of registers and spilled the accumulators (2-6 % slower).
template <int MODE>
__device__ __forceinline__ f32x16 mma32(const uint4& xa, const uint4& wb, const f32x16& c) {
  if constexpr (MODE != kDown)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wb),
                                                   __builtin_bit_cast(bf16x8, xa), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, xa),
                                                  __builtin_bit_cast(f16x8, wb), c, 0, 0, 0);
}

// WN: product columns per wave (128 or 64); a tile has BNB = 2 WN product
// columns.
template <int MODE, int WN, bool PACKED>
__global__ __launch_bounds__(kThreads, 1) void ffn_gemm_bf16(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int n_experts,
    int64_t cap_rows, const uint16_t* __restrict__ W, void* __restrict__ Cout, int K,
    int N_out, const float* __restrict__ dh_in, uint16_t* __restrict__ h_out,
    const uint16_t* const* __restrict__ w_ptrs, float* __restrict__ gu_out, int y_half,
    float* __restrict__ tail_ws, int ncus, int tail_cap) {
  constexpr bool GATED = MODE != kDown;  // gate and up columns paired in a wave
  constexpr int BM = bm_of(WN);
  constexpr int kTileA = BM * BK * 2;
  constexpr int NA = BM / 32;            // 1 KB activation copies per wave per step
  constexpr int BNB = 2 * WN;
  // Wave layout: 2 x 2 (two wave rows of BM / 2 rows, two wave columns of WN
  // product columns), or, for the down GEMM on wide tiles with packed
  // weights, 1 x 4: every wave all BM rows and WN / 2 product columns, so
  // each weight fragment is loaded by one wave only (with 2 x 2 both wave
  // rows load it) and every wave reads the whole activation tile from LDS.
  // Measured against 2 x 2 on one box: down GEMM -2 to -4 % on the
  // rank-share and skewed layers, unchanged on the Mixtral-style one; the
  // gate_up GEMM there +0.5 to 1.5 % (twice the LDS reads cost what the
  // weight loads save), so it keeps 2 x 2.
  constexpr int kWR = PACKED && WN == 128 && MODE == kDown ? 1 : 2;  // wave rows
  constexpr int WNW = BNB * kWR / 4;                // product columns per wave
  constexpr int kMaxMB = BM / (32 * kWR);           // 32-row blocks per wave
  constexpr int NQ = WNW / 32;                      // 32-column blocks per wave
  constexpr int ROWB = 2 * BNB;               // bytes per weight row in LDS
  constexpr int kTileB = BK * ROWB;
  constexpr int BN_OUT = GATED ? BNB / 2 : BNB;
  // Narrow tiles: one workgroup per CU works through several tiles, so the
  // tile table has LDS of its own. Wide tiles: one tile per workgroup, the
  // table lives in the staging memory until the first copy (a separate table
  // would cost the weight ring its third slot).
  constexpr bool kPersist = WN == 64;
  // LDS: activation ring of 2 tiles, then a weight ring of NSB tiles (and
  // the tile table). Packed weights go straight from memory to each wave's
  // registers: the LDS holds the activation ring only.
  constexpr int kTabInts = 2 * (kMaxTableExperts + 1);
  constexpr int kTab = kPersist ? kTabInts * 4 : 0;
  constexpr int NSA = 2;
  constexpr int NSB = PACKED ? 0 : (2 * kTileA + 3 * kTileB + kTab <= 160 * 1024 ? 3 : 2);
  constexpr int kLds = NSA * kTileA + NSB * kTileB;
  static_assert(kLds + kTab <= 160 * 1024, "LDS budget");
  static_assert(kTabInts * 4 <= (PACKED ? kTileA : kLds), "the table fits in the staging memory");
  // Packed weights: the two activation slots are separate arrays, so the
  // compiler can tell a copy into one slot from reads of the other and does
  // not wait for the copy before those reads.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[PACKED ? 16 : kLds];
  __shared__ __attribute__((aligned(1024))) unsigned char sA0[PACKED ? kTileA : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char sA1[PACKED ? kTileA : 16];
  __shared__ int s_tab[kPersist ? kTabInts : 1];
  int* s_pref = kPersist ? s_tab : reinterpret_cast<int*>(PACKED ? sA0 : smem);  // tiles before expert e
  int* s_off = s_pref + kMaxTableExperts + 1;  // first row of expert e (clamped to cap)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int NT = (N_out + BN_OUT - 1) / BN_OUT;
  const int ldw = GATED ? 2 * N_out : N_out;
  const int nk_all = K / BK;
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
  // Split-K tail (wide tiles, given a part buffer; the down GEMM, and the
  // gated GEMM with packed weights): one workgroup per CU runs at a time, so
  // R tiles take ceil(R / ncus) rounds and the last one runs rem = R mod ncus
  // tiles while the other CUs idle. Those rem tiles are cut along K into
  // n_parts parts (n_parts n_tail <= ncus: one short round); each part writes
  // its fp32 accumulators to tail_ws, with the tile's place in the output in
  // the header after the parts, and down_tail_finish_kernel (or, gated,
  // gate_tail_finish_kernel, which also applies the SiLU gate) adds each
  // tile's parts in part order and stores them. Tiles [0, n_whole) run whole.
  constexpr bool kSplit = !kPersist && (MODE == kDown || (MODE == kGateUp && PACKED));
  int n_whole = R, n_tail = 0, n_parts = 1;
  if constexpr (kSplit) {
    if (tail_ws != nullptr) {
      const int r = R % ncus;
      const int sp = r > 0 ? min(min(kMaxSplit, ncus / r), nk_all / min_split_steps<MODE>()) : 0;
      if (sp >= 2 && r * sp <= tail_cap) {
        n_whole = R - r;
        n_tail = r;
        n_parts = sp;
      }
    }
  }
  // Work items of this workgroup. Tiles [0, n_whole) are cut into 8
  // contiguous runs of ceil(n_whole / 8), run x served by the workgroups
  // b = x (mod 8) (the workgroups of XCD x); workgroup b takes tiles
  // x * per + b / 8 + i * G8 of the run, G8 = its XCD's workgroup count. One
  // tile each when the grid covers the tile list; several, one after
  // another, when the grid is one workgroup per CU. The workgroups past the
  // runs take the tail's parts (item n_whole + u: part u % n_parts of tail
  // tile u / n_parts).
  if (kSplit && tail_ws != nullptr && blockIdx.x == 0 && tid == 0) {
    int* hdr = reinterpret_cast<int*>(reinterpret_cast<char*>(tail_ws) +
                                      static_cast<int64_t>(tail_cap) * kDownPartBytes);
    hdr[0] = n_tail;
    hdr[1] = n_parts;
  }
  const int G8 = static_cast<int>(gridDim.x) / kXcds;
  const int xcd = static_cast<int>(blockIdx.x) % kXcds, slot = static_cast<int>(blockIdx.x) / kXcds;
  const int per = (n_whole + kXcds - 1) / kXcds;
  int it0 = xcd * per + slot, it_end = min((xcd + 1) * per, n_whole), it_step = G8;
  if (slot >= per) {
    const int u = (slot - per) * kXcds + xcd;
    it0 = n_whole + u;
    it_end = u < n_tail * n_parts ? it0 + 1 : it0;
    it_step = 1;
  }
  for (int it = it0; it < it_end; it += it_step) {
    // Item -> tile t and K-steps [kb, kb + nk). part: -1 a whole tile,
    // p >= 0 part p of a tail tile (its accumulators go to part unit
    // `unit`). (The names are distinct from the tile decode's locals below,
    // which the lambdas of the tile body would otherwise see instead.)
    int t = it, kb = 0, nk = nk_all, part = -1, unit = 0;
    if (it >= n_whole) {
      unit = it - n_whole;
      t = n_whole + unit / n_parts;
      part = unit % n_parts;
      kb = part * nk_all / n_parts;
      nk = (part + 1) * nk_all / n_parts - kb;
    }
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
    // An expert's tiles are ordered column block by column block over groups
    // of GR row blocks: all its row blocks in one group when it has at most 8
    // (then the workgroups an XCD runs at once share each weight tile and most
    // of the expert's activation rows), groups of 4 beyond that (a heavy
    // expert's concurrent tiles then span 4 row blocks x several column
    // blocks instead of many row blocks of one column block; measured on the
    // skewed 128-expert layer: gate_up GEMM -8 %, DRAM reads -7 to -18 %).
    const int GR = mt <= 8 ? mt : 4;
    const int full = mt / GR, in_full = full * GR * NT;
    int nb, mbk;
    if (local < in_full) {
      const int rg = local / (GR * NT), rem = local - rg * GR * NT;
      nb = rem / GR;
      mbk = rg * GR + (rem - nb * GR);
    } else {  // the last, partial group of gr < GR row blocks
      const int l2 = local - in_full, gr = mt - full * GR;
      nb = l2 / gr;
      mbk = full * GR + (l2 - nb * gr);
    }
    const int row_begin = seg_beg + mbk * chunk;
    const int rows = min(chunk, seg_end - row_begin);  // <= BM
    const int n0 = nb * BN_OUT;
    if (kSplit && part == 0 && tid == 0) {
      // the tail tile's place in the output, for down_tail_finish_kernel
      int4* hdr = reinterpret_cast<int4*>(reinterpret_cast<char*>(tail_ws) +
                                          static_cast<int64_t>(tail_cap) * kDownPartBytes);
      hdr[1 + (t - n_whole)] = make_int4(row_begin, max(rows, 0), n0, 0);
    }
    if (rows <= 0) continue;  // (uniform: the whole workgroup takes the same tile)
    if (!kPersist) __syncthreads();  // every wave has read the table

    // ---- copy assignment (global -> LDS), fixed for the tile ----
    // Activations: wave w copies the 8-row groups g = NA w + i (i < NA), rows
    // 8g .. 8g + 7; lane -> row 8g + (lane >> 3), LDS chunk lane & 7 (global
    // chunk swizzled). Rows past the segment lie past the buffer's end and read
    // as zeros. (Skipping whole groups past the segment instead makes the
    // compiler unswitch the K loop on that test, duplicating it with
    // accumulator copies.)
    // (both resources start at K-step kb: offsets within them count from it)
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + static_cast<int64_t>(row_begin) * K + kb * BK), 0, rows * K * 2 - kb * BK * 2,
        0x00020000);
    // Stacked experts ([n, K, ldw]) or one buffer per expert (w_ptrs[expert]);
    // packed weights hold 4 KB of fragments per column block and K-step.
    const uint16_t* wexp = w_ptrs ? w_ptrs[expert] : W + static_cast<int64_t>(expert) * K * ldw;
    const int b_skip = PACKED ? kb * 2048 : kb * BK * ldw;  // 16-bit elements
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(wexp + b_skip), 0, K * ldw * 2 - b_skip * 2, 0x00020000);
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
    // Bytes between consecutive K steps of one weight copy.
    const int b_step = BK * ldw * 2;
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_u8*)smem;

    // ---- compute assignment: wave (wm, wn) ----
    // 2 x 2: the tile's 32-row blocks holding rows of the segment are shared
    // out between the two wave rows (wm = 0 takes the first ceil(n/2)), so a
    // partial tile keeps both wave rows busy; 1 x 4: every wave takes all of
    // them. Wave wn owns product columns wn * WNW .. (for GEMM 1: gate columns
    // wn * WNW/2 .. and the same up columns).
    const int wm = kWR == 1 ? 0 : wave >> 1, wn = kWR == 1 ? wave : wave & 1;
    const int nblk = (rows + 31) / 32;
    const int nmb = kWR == 1 ? nblk : (wm == 0 ? (nblk + 1) / 2 : nblk / 2);
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
      const int blk = GATED ? ((q < NQ / 2 ? 0 : BNB / 2) + wn * (WNW / 2) + (q % (NQ / 2)) * 32)
                            : (wn * WNW + q * 32);
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
        const lds_u8* bbase = (const lds_u8*)smem + NSA * kTileA + sb * kTileB;
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
          acc[mb][q] = mma32<MODE>(fa[mb], fb[q], acc[mb][q]);
        }
      };
      // Copy item i of a step: activation copies 0..NA-1 first, then weight
      // copies NA..NA+NB-1. A step's items are spread over its 4 kMaxMB MFMA
      // groups so that the wave keeps the matrix core busy while the copies
      // issue.
      // A copy that is not needed (a step past the last) is still issued, with
      // an out-of-range offset, so it reads nothing and writes zeros into the
      // slot of a finished step; the select keeps the K loop free of branches.
      auto copy_item = [&](int i, bool do_a, int kt_a, int slot_a, bool do_b, int kt_b,
                           int slot_b) {
        if (i < NA) {
          dma16(a_rsrc, do_a ? a_voff[i] : kOutOfRange, kt_a * BK * 2,
                lds0 + slot_a * kTileA + (wave * NA + i) * 1024);
        } else if (i - NA < NB) {
          dma16(b_rsrc, do_b ? b_voff[i - NA] : kOutOfRange, kt_b * b_step,
                lds0 + NSA * kTileA + slot_b * kTileB + (wave * NB + i - NA) * 1024);
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
        // Every step issues all of its copies; those for steps past the last
        // get an out-of-range offset (copy_item), so the loop has no branch
        // around them: measured on stacked weights, Mixtral-style gate_up
        // 3567-3579 -> 3507-3512 us and down 2119-2154 -> 2081-2105 us.
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
    // Packed weights: fragment (wave column block q, slice kk of step kt) is
    // the 16 bytes of this lane at bd_off[q] + (4 kt + kk) KB of the packed
    // expert weight (columns past N_out read as zeros).
    int bd_off[NQ];
  #pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c0 = n0 + (GATED ? wn * (WNW / 2) + (q % (NQ / 2)) * 32 : wn * WNW + q * 32);
      const int cb = ((GATED && q >= NQ / 2 ? N_out : 0) + c0) >> 5;
      bd_off[q] = c0 < N_out ? cb * (K >> 4) * 1024 + lane * 16 : kOutOfRange;
    }
    // Narrow tiles (320 x 128): each step starts with the barrier and all of
    // the step's activation copies, then runs its 4 K-slices. (The wide
    // tiles' loop below, with the copies spread over a step's last slice,
    // measured 5 % slower here: a narrow step has 10 copies per wave against
    // 10 MFMAs in that slice, and their issue stalls the matrix core.)
    auto run_direct_narrow = [&](auto nmb_c) {
      constexpr int NMB = decltype(nmb_c)::value;
      // Weights of one step in registers, fb[kk][q]. Step kt + 1's slice-kk
      // fragments are loaded right after step kt's slice-kk MFMAs have read
      // fb[kk] (a whole step to arrive). Loads and copies are compiler
      // builtins, so the compiler counts all of them and waits for each
      // weight load exactly before its first use; the two activation slots
      // are separate arrays read at fixed slots (the loop runs steps in
      // pairs), so it can tell a copy into one slot from reads of the other.
      uint4 fb[4][NQ];
      auto load_b = [&](int kt, int kk, int pad) {
  #pragma unroll
        for (int q = 0; q < NQ; ++q)
        {
          const int voff = bd_off[q] + pad + kk * 1024;
          fb[kk][q] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, voff, kt * 4096, 0));
        }
      };
      typedef __attribute__((address_space(3))) void lds_void;
      auto copy_a = [&](int kt, unsigned char* slot, int pad) {
  #pragma unroll
        for (int i = 0; i < NA; ++i) {
          // (the offset goes through a local: with the array element written
          // in the call, the host pass drops the kernel's launch stub)
          const int voff = a_voff[i] + pad;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              a_rsrc, (lds_void*)(slot + (wave * NA + i) * 1024), 16, voff, kt * BK * 2, 0, 0);
        }
      };
      auto mfma_row = [&](int mb, const uint4(&fa)[kMaxMB], const uint4(&fbk)[NQ]) {
  #pragma unroll
        for (int q = 0; q < NQ; ++q) {
          acc[mb][q] = mma32<MODE>(fa[mb], fbk[q], acc[mb][q]);
        }
      };
      // Issue order: prologue A(0), B(0); step kt: A(kt + 1) at its start,
      // then B(kt + 1) slice by slice. An odd step count is padded with one
      // step whose loads (and those made for the step after the last) are
      // out of range, so they read zeros and its MFMAs add nothing.
      // (in slice order, as the steps issue them, so that the compiler's
      // count at the loop head matches the steady state's)
      copy_a(0, sA0, 0);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        load_b(0, kk, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      auto step = [&](int kt, const unsigned char* cur, unsigned char* fill) {
        // Wait for this wave's A(kt) copies: only B(kt) (4 NQ loads, issued in
        // step kt - 1 or the prologue) came after them (loads complete in
        // issue order). The barrier then makes every wave's copies visible and
        // ends step kt - 1, whose slot A(kt + 1) overwrites.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * NQ));
        __builtin_amdgcn_s_barrier();
        const int pad = kt + 1 < nk ? 0 : kOutOfRange;
        copy_a(kt + 1, fill, pad);
        __builtin_amdgcn_sched_barrier(0);
        uint4 fa[2][kMaxMB];
  #pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          fa[0][mb] = *reinterpret_cast<const uint4*>(cur + a_addr[0] + mb * 32 * 128);
  #pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (kk < 3) {
  #pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
              fa[(kk + 1) & 1][mb] =
                  *reinterpret_cast<const uint4*>(cur + a_addr[kk + 1] + mb * 32 * 128);
          }
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int mb = 0; mb < kMaxMB; ++mb)
            if (mb < NMB) mfma_row(mb, fa[kk & 1], fb[kk]);
          __builtin_amdgcn_sched_barrier(0);
          load_b(kt + 1, kk, pad);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      for (int kt = 0; kt < nk; kt += 2) {
        step(kt, sA0, sA1);
        step(kt + 1, sA1, sA0);
      }
      // the last step's loads (of the step after it) are still in flight
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    };
    // Wide tiles (256 x 256).
    auto run_direct = [&](auto nmb_c) {
      constexpr int NMB = decltype(nmb_c)::value;
      // A 64-deep step kt is 4 K-slices kk of NMB x NQ MFMAs per wave.
      // Weights go straight to registers one step ahead: fragment (kk, q) of
      // step kt + 1 is loaded into fb[kk][q] as soon as step kt's MFMAs have
      // read it. Activations are copied to LDS two steps ahead (two slots) and
      // read into fa[kk & 1] one slice ahead. A step's one barrier sits before
      // its last slice: by then every wave's copy of A(kt + 1) has landed and
      // every wave holds its last fragments of A(kt) in registers, so the copy
      // of A(kt + 2) may overwrite that slot, and the first fragments of step
      // kt + 1 are read while the last slice multiplies: the next step starts
      // without a barrier or a read latency. The loads are spread between the
      // MFMAs (after each column block's MFMAs: that block's next weight
      // fragment and a share of the copies; after the first block, the
      // fragment reads of the next slice), so each issues while the matrix
      // core works (measured on the Mixtral-style layer: gate_up GEMM -6 %,
      // down GEMM on these tiles -4 %; reading at the start of a slice
      // instead was 1 % slower). Loads and copies are compiler builtins, so the compiler counts all of them and
      // waits for each exactly before its first use; the two activation slots
      // are separate arrays used at fixed slots (the loop runs steps in
      // pairs), so it can tell a copy into one slot from reads of the other.
      uint4 fb[4][NQ];
      uint4 fa[2][kMaxMB];
      auto load_b = [&](int kt, int kk, int q, int pad) {
        const int voff = bd_off[q] + pad + kk * 1024;
        fb[kk][q] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, voff, kt * 4096, 0));
      };
      typedef __attribute__((address_space(3))) void lds_void;
      auto copy_a = [&](int kt, unsigned char* slot, int i, int pad) {
        // (the offset goes through a local: with the array element written
        // in the call, the host pass drops the kernel's launch stub)
        const int voff = a_voff[i] + pad;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (lds_void*)(slot + (wave * NA + i) * 1024), 16, voff, kt * BK * 2, 0, 0);
      };
      auto read_a = [&](const unsigned char* slot, int kk, uint4(&dst)[kMaxMB]) {
  #pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          dst[mb] = *reinterpret_cast<const uint4*>(slot + a_addr[kk] + mb * 32 * 128);
      };
      auto mfma_col = [&](int q, const uint4(&fak)[kMaxMB], const uint4& fbq) {
  #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          acc[mb][q] = mma32<MODE>(fak[mb], fbq, acc[mb][q]);
        }
      };
      // Issue order, the same in the prologue and in every step (so that the
      // compiler's counts at the loop head match): B(kt, 0..2), A(kt + 1),
      // B(kt, 3). An odd step count is padded with one step whose loads (and
      // those made for the steps after the last) are out of range: they read
      // zeros and its MFMAs add nothing.
  #pragma unroll
      for (int i = 0; i < NA; ++i) copy_a(0, sA0, i, 0);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int kk = 0; kk < 3; ++kk) {
  #pragma unroll
        for (int q = 0; q < NQ; ++q) load_b(0, kk, q, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        const int pad1 = nk > 1 ? 0 : kOutOfRange;
  #pragma unroll
        for (int i = 0; i < NA; ++i) copy_a(1, sA1, i, pad1);
      }
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int q = 0; q < NQ; ++q) load_b(0, 3, q, 0);
      __builtin_amdgcn_sched_barrier(0);
      // This wave's copies of A(0) are done (only B(0, 0..2), A(1) and B(0, 3)
      // may be outstanding); after the barrier every wave's are.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * NQ + NA));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_a(sA0, 0, fa[0]);
      __builtin_amdgcn_sched_barrier(0);
      auto step = [&](int kt, unsigned char* cur, const unsigned char* nxt) {
        const int pad_b = kt + 1 < nk ? 0 : kOutOfRange;  // weights of step kt + 1
        const int pad_a = kt + 2 < nk ? 0 : kOutOfRange;  // activations of step kt + 2
  #pragma unroll
        for (int kk = 0; kk < 3; ++kk) {
  #pragma unroll
          for (int q = 0; q < NQ; ++q) {
            mfma_col(q, fa[kk & 1], fb[kk][q]);
            __builtin_amdgcn_sched_barrier(0);
            load_b(kt + 1, kk, q, pad_b);
            if (q == 0) read_a(cur, kk + 1, fa[(kk + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // This wave's copies of A(kt + 1) are done (after them only B(kt, 3)
        // and B(kt + 1, 0..2) were issued) and its reads of A(kt) have
        // returned; after the barrier the same holds for every wave.
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(4 * NQ));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int q = 0; q < NQ; ++q) {
          mfma_col(q, fa[1], fb[3][q]);
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int i = q * NA / NQ; i < (q + 1) * NA / NQ; ++i) copy_a(kt + 2, cur, i, pad_a);
          if (q == 0) read_a(nxt, 0, fa[0]);
          __builtin_amdgcn_sched_barrier(0);
        }
  #pragma unroll
        for (int q = 0; q < NQ; ++q) load_b(kt + 1, 3, q, pad_b);
        __builtin_amdgcn_sched_barrier(0);
      };
      for (int kt = 0; kt < nk; kt += 2) {
        step(kt, sA0, sA1);
        step(kt + 1, sA1, sA0);
      }
      // the last steps' loads (of the steps after them) are still in flight
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    };
    // kGateUpBwd: the epilogue's dH values of row block 0 are loaded before
    // the K loop (issued ahead of its copies, so the copies' vmcnt waits also
    // cover them); those of row block mb + 1 while block mb is computed.
    constexpr int NQD = MODE == kGateUpBwd ? NQ / 2 : 1;
    float4 dpre[2][NQD][4];
    // (rows past the segment lie past the resource and read as zeros; so do
    // columns past N_out, given an out-of-range offset)
    const __amdgpu_buffer_rsrc_t dh_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(dh_in + (MODE == kGateUpBwd ? static_cast<int64_t>(row_begin) * N_out : 0)), 0,
        MODE == kGateUpBwd ? rows * N_out * 4 : 0, 0x00020000);
    auto load_dh = [&](int mb, float4(&d)[NQD][4]) {
      const int r = rowbase + mb * 32 + (lane & 31);
  #pragma unroll
      for (int q = 0; q < NQD; ++q) {
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn * (WNW / 2) + q * 32 + 8 * g + 4 * half;
          const int voff = col < N_out ? (r * N_out + col) * 4 : kOutOfRange;
          d[q][g] = __builtin_bit_cast(
              float4, __builtin_amdgcn_raw_buffer_load_b128(dh_rsrc, voff, 0, 0));
        }
      }
    };
    if (MODE == kGateUpBwd && nmb > 0) load_dh(0, dpre[0]);
    static_assert(PACKED || (kMaxMB <= 5 && NA + NB <= 4 * kMaxMB),
                  "copy items fit the MFMA groups");
    // The epilogue is instantiated per row-block count, next to the K loop
    // that filled the accumulators, so they stay in their registers until
    // read (with one epilogue after the switch, the compiler copied all of
    // them out at the join and spilled).
    auto epilogue = [&](auto nmb_c) {
      constexpr int NMB = decltype(nmb_c)::value;
      // ---- epilogue of the gated GEMMs ----
      // Register 4 g + i of lane l holds row l % 32 and column
      // 8 g + 4 (l / 32) + i of its 32x32 block (see mma32): each store writes
      // 4 adjacent columns of one row, 8 (bf16, fp16) or 16 (fp32) bytes.
      // Stores go through buffer resources over the tile's rows of each
      // output: a row past the segment lies past the resource and a column
      // past N_out gets an out-of-range offset, the hardware drops such
      // stores, and the epilogue is one straight run of code (a branch around
      // each store made the compiler copy all accumulators out at once and
      // spill). Offsets stay below 2^30: at most 256 rows of 8 N_out bytes,
      // N_out <= 2^18.
      auto out_rsrc = [&](void* base, int pitch) {
        return __builtin_amdgcn_make_buffer_rsrc(
            static_cast<char*>(base) + static_cast<int64_t>(row_begin) * pitch, 0, rows * pitch,
            0x00020000);
      };
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
      const int cpitch = (MODE == kGateUpBwd ? 2 * N_out : N_out) * 2;
      const __amdgpu_buffer_rsrc_t c_rsrc = out_rsrc(Cout, cpitch);
      const __amdgpu_buffer_rsrc_t h_rsrc =
          out_rsrc(MODE == kGateUpBwd ? static_cast<void*>(h_out) : Cout, N_out * 2);
      const __amdgpu_buffer_rsrc_t gu_rsrc =
          out_rsrc(MODE == kGateUpSave ? static_cast<void*>(gu_out) : Cout, N_out * 8);
    #pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        if (MODE == kGateUpBwd && mb + 1 < NMB) load_dh(mb + 1, dpre[(mb + 1) & 1]);
        const int r = rowbase + mb * 32 + (lane & 31);  // row within the tile
    #pragma unroll
        for (int q = 0; q < NQ / 2; ++q) {
    #pragma unroll
          for (int g = 0; g < 4; ++g) {
            // (one group of 4 columns at a time: left to itself the scheduler
            // reads all accumulators first and runs out of registers)
            __builtin_amdgcn_sched_barrier(0);
            const int col = n0 + wn * (WNW / 2) + q * 32 + 8 * g + 4 * half;
            const bool col_ok = col < N_out;
            float gv[4], uv[4];
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
              gv[i] = acc[mb][q][4 * g + i];
              uv[i] = acc[mb][q + NQ / 2][4 * g + i];
            }
            if (MODE == kGateUpBwd) {
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
              const int og = col_ok ? (r * 2 * N_out + col) * 2 : kOutOfRange;
              const int oh = col_ok ? (r * N_out + col) * 2 : kOutOfRange;
              __builtin_amdgcn_raw_buffer_store_b64(u32x2{dgw[0], dgw[1]}, c_rsrc, og, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b64(u32x2{duw[0], duw[1]}, c_rsrc, og + N_out * 2, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b64(u32x2{hw[0], hw[1]}, h_rsrc, oh, 0, 0);
            } else {
              // H = SiLU(G) U from the same accumulator values in both forward
              // modes, so the training forward's H (and y) is the plain
              // forward's, bit for bit.
              if (MODE == kGateUpSave) {
                const int o = col_ok ? (r * 2 * N_out + col) * 4 : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, make_float4(gv[0], gv[1], gv[2], gv[3])), gu_rsrc, o, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, make_float4(uv[0], uv[1], uv[2], uv[3])), gu_rsrc,
                    o + N_out * 4, 0, 0);
              }
              float v[4];
    #pragma unroll
              for (int i = 0; i < 4; ++i)
                // SiLU(g) u = g u / (1 + exp(-g)), exp via exp2, then reciprocal
                v[i] = gv[i] * uv[i] *
                       __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gv[i]));
              const int o = col_ok ? (r * N_out + col) * 2 : kOutOfRange;
              __builtin_amdgcn_raw_buffer_store_b64(
                  u32x2{f16_sat_bits(v[0]) | (f16_sat_bits(v[1]) << 16),
                        f16_sat_bits(v[2]) | (f16_sat_bits(v[3]) << 16)},
                  c_rsrc, o, 0, 0);
            }
          }
        }
      }
    };
    // A tail part's accumulators in tail_ws, 256 KB per unit (tail tile
    // unit / n_parts, part unit % n_parts), in the tile's own block order
    // whatever the wave layout: [unit][row block][column block][g][lane] x
    // float4 (8 x 8 blocks of 32 x 32), each float4 holding accumulator
    // registers 4 g .. 4 g + 3 of the block.
    constexpr int kPartF4 = (BM / 32) * (BNB / 32) * 4 * 64;
    static_assert(kPersist || kPartF4 * 16 == kDownPartBytes, "part size");
    auto go = [&](auto nmb_c) {
      constexpr int NMB = decltype(nmb_c)::value;
      if constexpr (PACKED && WN == 128)
        run_direct(nmb_c);
      else if constexpr (PACKED)
        run_direct_narrow(nmb_c);
      else
        run(nmb_c);
      if (kSplit && part >= 0) {
        if constexpr (MODE == kDown) {
          float4* pw = reinterpret_cast<float4*>(tail_ws) +
                       static_cast<int64_t>(unit) * kPartF4 +
                       (((rowbase >> 5) * (BNB / 32) + wn * NQ) * 4) * 64 + lane;
  #pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
  #pragma unroll
            for (int q = 0; q < NQ; ++q)
  #pragma unroll
              for (int g = 0; g < 4; ++g)
                pw[((mb * (BNB / 32) + q) * 4 + g) * 64] =
                    make_float4(acc[mb][q][4 * g], acc[mb][q][4 * g + 1], acc[mb][q][4 * g + 2],
                                acc[mb][q][4 * g + 3]);
        } else {
          // Gated: through a buffer resource (one lane offset, each block's
          // offset a scalar); with a 64-bit address per store, as above, the
          // kernel ran out of registers and spilled in its epilogue.
          typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
          const __amdgpu_buffer_rsrc_t p_rsrc = __builtin_amdgcn_make_buffer_rsrc(
              reinterpret_cast<char*>(tail_ws) + static_cast<int64_t>(unit) * kDownPartBytes, 0,
              static_cast<int>(kDownPartBytes), 0x00020000);
          const int p_voff = ((((rowbase >> 5) * (BNB / 32) + wn * NQ) * 4) * 64 + lane) * 16;
  #pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
  #pragma unroll
            for (int q = 0; q < NQ; ++q)
  #pragma unroll
              for (int g = 0; g < 4; ++g)
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4{__float_as_uint(acc[mb][q][4 * g]),
                          __float_as_uint(acc[mb][q][4 * g + 1]),
                          __float_as_uint(acc[mb][q][4 * g + 2]),
                          __float_as_uint(acc[mb][q][4 * g + 3])},
                    p_rsrc, p_voff, ((mb * (BNB / 32) + q) * 4 + g) * 64 * 16, 0);
        }
        return;
      }
      if constexpr (MODE != kDown && NMB > 0) epilogue(nmb_c);
    };
    switch (nmb) {
      case 8:  // 1 x 4 layout only
        if constexpr (kMaxMB >= 8) go(std::integral_constant<int, 8>{});
        break;
      case 7:
        if constexpr (kMaxMB >= 7) go(std::integral_constant<int, 7>{});
        break;
      case 6:
        if constexpr (kMaxMB >= 6) go(std::integral_constant<int, 6>{});
        break;
      case 5:  // 1 x 4, or 2 x 2 narrow tiles (2 x 2 wide tiles give nmb <= 4)
        if constexpr (kMaxMB >= 5) go(std::integral_constant<int, 5>{});
        break;
      case 4: go(std::integral_constant<int, 4>{}); break;
      case 3: go(std::integral_constant<int, 3>{}); break;
      case 2: go(std::integral_constant<int, 2>{}); break;
      case 1: go(std::integral_constant<int, 1>{}); break;
      default: go(std::integral_constant<int, 0>{}); break;
    }
    if (MODE == kDown && nmb > 0 && part < 0) {
      // ---- epilogue of the down GEMM ----
      // Accumulator register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4
      // and column l % 32 of its 32x32 block. A 4x4 transpose inside each group of
      // 4 lanes (two DPP exchange rounds) gives every lane 4 adjacent columns of
      // one row, so each store writes 8 (fp16) or 16 (fp32) bytes. Y is fp32,
      // or (y_half) fp16 rounded to nearest even and saturated at +-65504 like H.
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
    #pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int col = n0 + wn * WNW + q * 32 + (lane & 28);
    #pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int row = row_begin + rowbase + mb * 32 + 8 * g + 4 * half + quad;
            float v[4];
    #pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[mb][q][4 * g + i];
            transpose4(v);
            if (row < row_end && col < N_out) {
              const int64_t o = static_cast<int64_t>(row) * N_out + col;
              if (y_half)
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Cout) + o) =
                    make_uint2(f16_sat_bits(v[0]) | (f16_sat_bits(v[1]) << 16),
                               f16_sat_bits(v[2]) | (f16_sat_bits(v[3]) << 16));
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

// Second pass of the down GEMM's split-K tail: adds each tail tile's parts
// (written by ffn_gemm_bf16<kDown, 128> in part order, 0 + p0 + p1 + ...) and
// stores Y like the GEMM's epilogue (fp32, or fp16 rounded to nearest even
// and saturated). One workgroup per (tail tile, 32-row block, half of the 8
// column blocks): thread (q, lane) sums the float4s of column block
// 4 half + q and lane, i.e. rows 8 g + 4 (lane / 32) + i and column lane % 32
// of the 32 x 32 block (the down GEMM's accumulator order). The header after
// the parts gives the tail size and part count, and each tail tile's first
// row, rows and first column; workgroups past the tail or its rows exit.
__global__ __launch_bounds__(256) void down_tail_finish_kernel(const float4* __restrict__ parts,
                                                              const int4* __restrict__ hdr,
                                                              void* __restrict__ y, int N_out,
                                                              int y_half) {
  constexpr int kBlocks = 8;  // 32-row (and 32-column) blocks of a 256 x 256 tile
  const int n_tail = hdr[0].x, n_parts = hdr[0].y;
  const int tile = blockIdx.x / 16, mb = (blockIdx.x / 2) % kBlocks, qh = blockIdx.x % 2;
  if (tile >= n_tail) return;
  const int4 h = hdr[1 + tile];  // row_begin, rows, n0
  if (mb * 32 >= h.y) return;
  const int q = qh * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = h.z + q * 32 + (lane & 31);
  const int row_end = h.x + h.y;
  for (int g = 0; g < 4; ++g) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = 0; p < n_parts; ++p) {
      const int64_t u = static_cast<int64_t>(tile) * n_parts + p;
      const float4 w = parts[(((u * kBlocks + mb) * kBlocks + q) * 4 + g) * 64 + lane];
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    const float vals[4] = {v.x, v.y, v.z, v.w};
    for (int i = 0; i < 4; ++i) {
      const int row = h.x + mb * 32 + 8 * g + 4 * (lane >> 5) + i;
      if (row >= row_end || col >= N_out) continue;
      const int64_t o = static_cast<int64_t>(row) * N_out + col;
      if (y_half)
        static_cast<uint16_t*>(y)[o] = static_cast<uint16_t>(f16_sat_bits(vals[i]));
      else
        static_cast<float*>(y)[o] = vals[i];
    }
  }
}

// Second pass of the gated GEMM's split-K tail (packed weights, 2 x 2 waves):
// adds each tail tile's parts in part order, 0 + p0 + p1 + ..., for the gate
// and the up pre-activations and stores H = SiLU(G) U like the GEMM's
// epilogue (the same arithmetic, fp16 rounded to nearest even and
// saturated). One workgroup per (tail tile, 32-row block): thread (wn, q,
// lane) takes the tile's gate column block 4 wn + q and up column block
// 4 wn + q + 2 (the blocks wave column wn holds), whose registers 4 g + i
// of lane l are row l % 32 and column 8 g + 4 (l / 32) + i of a 32 x 32
// block (the gated GEMMs' transposed accumulator order).
__global__ __launch_bounds__(256) void gate_tail_finish_kernel(const float4* __restrict__ parts,
                                                              const int4* __restrict__ hdr,
                                                              uint16_t* __restrict__ h,
                                                              int N_out) {
  constexpr int kBlocks = 8;  // 32-row (and 32-column) blocks of a 256 x 256 tile
  const int n_tail = hdr[0].x, n_parts = hdr[0].y;
  const int tile = blockIdx.x / kBlocks, mb = blockIdx.x % kBlocks;
  if (tile >= n_tail) return;
  const int4 hh = hdr[1 + tile];  // row_begin, rows, n0 (first H column)
  const int wn = threadIdx.x >> 7, q = (threadIdx.x >> 6) & 1, lane = threadIdx.x & 63;
  const int row = mb * 32 + (lane & 31);
  if (row >= hh.y) return;
  const int qg = 4 * wn + q, qu = qg + 2;
  for (int g = 0; g < 4; ++g) {
    float gv[4] = {0.f, 0.f, 0.f, 0.f}, uv[4] = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < n_parts; ++p) {
      const int64_t u = static_cast<int64_t>(tile) * n_parts + p;
      const float4 a = parts[(((u * kBlocks + mb) * kBlocks + qg) * 4 + g) * 64 + lane];
      const float4 b = parts[(((u * kBlocks + mb) * kBlocks + qu) * 4 + g) * 64 + lane];
      gv[0] += a.x; gv[1] += a.y; gv[2] += a.z; gv[3] += a.w;
      uv[0] += b.x; uv[1] += b.y; uv[2] += b.z; uv[3] += b.w;
    }
    const int col = hh.z + 64 * wn + 32 * q + 8 * g + 4 * (lane >> 5);
    if (col >= N_out) continue;
    float v[4];
    for (int i = 0; i < 4; ++i)
      v[i] = gv[i] * uv[i] *
             __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gv[i]));
    *reinterpret_cast<uint2*>(h + static_cast<int64_t>(hh.x + row) * N_out + col) =
        make_uint2(f16_sat_bits(v[0]) | (f16_sat_bits(v[1]) << 16),
                   f16_sat_bits(v[2]) | (f16_sat_bits(v[3]) << 16));
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
// takes about 0.73 of a wide one's time (256 x 256; measured on the packed
// grouped GEMMs: 0.69 for the worked-example gate_up GEMM, 0.79 for the
// Mixtral-style down GEMM, whose wide tiles then win 1.80 ms to 1.99 ms).
// kWideOut: output columns of a wide tile (128 gated, 256 for the down GEMM).
bool choose_wide(int n_experts, int64_t cap_rows, int n_out, bool has_offsets, int kWideOut) {
  const int64_t ne = has_offsets ? n_experts : 1;
  const double mean = static_cast<double>(cap_rows) / static_cast<double>(ne);
  const double sd = has_offsets ? std::sqrt(mean) : 0.0;
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
  return 100 * waves_w <= 73 * waves_n;
}

template <int MODE, bool PACKED = false>
hipError_t launch_ffn(int n_experts, int64_t cap_rows, int K, int n_out, const void* a,
                      const int32_t* offsets, const void* w, void* out, hipStream_t s,
                      const float* dh_in = nullptr, void* h_out = nullptr,
                      const void* const* w_ptrs = nullptr, float* gu_out = nullptr,
                      bool y_half = false, float* tail_ws = nullptr, int tail_cap = 0) {
  constexpr int kWideOut = MODE != kDown ? 128 : 256;
  if (choose_wide(n_experts, cap_rows, n_out, offsets != nullptr, kWideOut)) {
    const int64_t tiles = tile_bound(cap_rows, offsets, n_experts, n_out, kWideOut, bm_of(128));
    const int cus = std::max(kXcds, num_cus() / kXcds * kXcds);
    // With a part buffer the tail may be split along K (the down GEMM, and
    // the gated GEMM on packed weights): the grid then has room for the parts
    // (at most cus more workgroups than tiles), and a second launch sums them.
    constexpr bool kCanSplit = MODE == kDown || (MODE == kGateUp && PACKED);
    const bool split = kCanSplit && tail_ws != nullptr && tail_cap > 0 &&
                       K / BK >= 2 * min_split_steps<MODE>();
    const unsigned g = grid_of(tiles + (split ? cus : 0), false);
    ffn_gemm_bf16<MODE, 128, PACKED><<<g, kThreads, 0, s>>>(
        static_cast<const uint16_t*>(a), offsets, n_experts, cap_rows,
        static_cast<const uint16_t*>(w), out, K, n_out, dh_in, static_cast<uint16_t*>(h_out),
        reinterpret_cast<const uint16_t* const*>(w_ptrs), gu_out, y_half ? 1 : 0,
        split ? tail_ws : nullptr, cus, tail_cap);
    if (split) {
      // at most tail_cap / 2 tail tiles (2 parts or more each)
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int4* hdr = reinterpret_cast<const int4*>(
          reinterpret_cast<char*>(tail_ws) + static_cast<int64_t>(tail_cap) * kDownPartBytes);
      if (MODE == kDown)  // 16 workgroups per tile
        down_tail_finish_kernel<<<static_cast<unsigned>(tail_cap / 2 * 16), 256, 0, s>>>(
            reinterpret_cast<const float4*>(tail_ws), hdr, out, n_out, y_half ? 1 : 0);
      else  // 8 workgroups per tile
        gate_tail_finish_kernel<<<static_cast<unsigned>(tail_cap / 2 * 8), 256, 0, s>>>(
            reinterpret_cast<const float4*>(tail_ws), hdr, static_cast<uint16_t*>(out), n_out);
    }
  } else {
    const unsigned g =
        grid_of(tile_bound(cap_rows, offsets, n_experts, n_out, kWideOut / 2, bm_of(64)), true);
    ffn_gemm_bf16<MODE, 64, PACKED><<<g, kThreads, 0, s>>>(static_cast<const uint16_t*>(a), offsets,
                                                   n_experts, cap_rows,
                                                   static_cast<const uint16_t*>(w), out, K, n_out,
                                                   dh_in, static_cast<uint16_t*>(h_out),
                                                   reinterpret_cast<const uint16_t* const*>(w_ptrs),
                                                   gu_out, y_half ? 1 : 0, nullptr, 0, 0);
  }
  return hipGetLastError();
}

}  // namespace

void ffn_tile_shape_bf16(int n_experts, int64_t cap_rows, int D, int inter, bool has_offsets,
                         int gemm, int* rows, int* cols) {
  const int kWideOut = gemm == 0 ? 128 : 256;
  const bool wide = choose_wide(n_experts, cap_rows, gemm == 0 ? inter : D, has_offsets, kWideOut);
  *rows = bm_of(wide ? 128 : 64);
  *cols = wide ? 256 : 128;  // product columns (gate + up for the gated GEMM)
}

// Part-buffer units in tail_bytes bytes (0 without a buffer).
static int tail_units(const void* tail_ws, size_t tail_bytes) {
  return tail_ws && tail_bytes > kTailHeaderBytes
             ? static_cast<int>((tail_bytes - kTailHeaderBytes) / kDownPartBytes)
             : 0;
}

hipError_t launch_gate_up_bf16(int n_experts, int64_t cap_rows, int D, int inter,
                               const void* x_perm, const int32_t* offsets, const void* w_gate_up,
                               void* h, hipStream_t s, const void* const* w_ptrs, bool packed,
                               void* tail_ws, size_t tail_bytes) {
  if (cap_rows == 0) return hipSuccess;
  if (packed)
    return launch_ffn<kGateUp, true>(n_experts, cap_rows, D, inter, x_perm, offsets, w_gate_up,
                                     h, s, nullptr, nullptr, w_ptrs, nullptr, false,
                                     static_cast<float*>(tail_ws), tail_units(tail_ws, tail_bytes));
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
                            const void* const* w_ptrs, bool packed, bool y_half, void* tail_ws,
                            size_t tail_bytes) {
  if (cap_rows == 0) return hipSuccess;
  float* tw = static_cast<float*>(tail_ws);
  const int cap = tail_units(tail_ws, tail_bytes);
  if (packed)
    return launch_ffn<kDown, true>(n_experts, cap_rows, inter, D, h, offsets, w_down, y, s,
                                   nullptr, nullptr, w_ptrs, nullptr, y_half, tw, cap);
  return launch_ffn<kDown>(n_experts, cap_rows, inter, D, h, offsets, w_down, y, s, nullptr,
                           nullptr, w_ptrs, nullptr, y_half, tw, cap);
}

size_t down_tail_bytes(int64_t cap_rows, int n_experts, int D) {
  const int64_t tiles = ((cap_rows + 255) / 256 + n_experts) * ((D + 255) / 256);
  return static_cast<size_t>(std::min<int64_t>(kMaxTailUnits, kMaxSplit * tiles)) * kDownPartBytes +
         kTailHeaderBytes;
}

size_t gate_up_tail_bytes(int64_t cap_rows, int n_experts, int inter) {
  const int64_t tiles = ((cap_rows + 255) / 256 + n_experts) * ((inter + 127) / 128);
  return static_cast<size_t>(std::min<int64_t>(kMaxTailUnits, kMaxSplit * tiles)) * kDownPartBytes +
         kTailHeaderBytes;
}

// Packs stacked expert weights w [n][K][N] (16-bit) into the grouped GEMMs'
// operand order: out[e][cb][ks][l][j] = w[e][16 ks + 8 (l / 32) + j][32 cb + l % 32]
// for 32-column block cb, 16-deep K slice ks, lane l, j < 8 (one 16-byte
// chunk per lane, 1 KB per fragment). TO_F16: each bf16 value converted to
// fp16, rounding to nearest even (the conversion the stacked down GEMM does
// after its LDS reads, so both layouts multiply the same values).
template <bool TO_F16>
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ w,
                                                           uint4* __restrict__ out, int64_t n_chunks,
                                                           int K, int N) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= n_chunks) return;
  const int64_t per_e = static_cast<int64_t>(K) * N / 8;  // chunks per expert
  const int64_t e = gid / per_e, r = gid - e * per_e;
  const int lane = static_cast<int>(r & 63);
  const int64_t frag = r >> 6;
  const int nks = K >> 4;
  const int ks = static_cast<int>(frag % nks), cb = static_cast<int>(frag / nks);
  const int k0 = 16 * ks + 8 * (lane >> 5), col = 32 * cb + (lane & 31);
  const uint16_t* src = w + e * K * N + static_cast<int64_t>(k0) * N + col;
  uint32_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t pair = static_cast<uint32_t>(src[(2 * i) * static_cast<int64_t>(N)]) |
                          (static_cast<uint32_t>(src[(2 * i + 1) * static_cast<int64_t>(N)]) << 16);
    v[i] = TO_F16 ? bf16x2_to_f16x2(pair) : pair;
  }
  out[gid] = make_uint4(v[0], v[1], v[2], v[3]);
}

hipError_t launch_pack_weights(int n, int K, int N, bool to_f16, const void* w, void* out,
                               hipStream_t s) {
  const int64_t chunks = static_cast<int64_t>(n) * K * N / 8;
  if (chunks == 0) return hipSuccess;
  const unsigned g = static_cast<unsigned>((chunks + 255) / 256);
  if (to_f16)
    pack_weights_kernel<true><<<g, 256, 0, s>>>(static_cast<const uint16_t*>(w),
                                               static_cast<uint4*>(out), chunks, K, N);
  else
    pack_weights_kernel<false><<<g, 256, 0, s>>>(static_cast<const uint16_t*>(w),
                                                static_cast<uint4*>(out), chunks, K, N);
  return hipGetLastError();
}

}  // namespace moe
