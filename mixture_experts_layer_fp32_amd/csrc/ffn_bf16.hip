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
// the bf16 down_proj tile converted to fp16 while it is staged into LDS
// (exact for |w| in [2^-14, 65504]). Y is written in fp32 and rounded once,
// at the combine.
//
// Tiling: a 256-thread workgroup computes a 128-row x 256-column block of
// products over K in steps of 64. For GEMM 1 the 256 columns are 128 gate
// columns and the 128 matching up columns, so the SiLU-gate epilogue pairs
// them in registers and writes 128 columns of H. Each wavefront owns 64 rows
// x 128 product columns = 2 x 4 tiles of v_mfma_f32_32x32x16.
//
// LDS layouts (double-buffered; the global loads of the next K-step are in
// flight while the current one is multiplied):
//  * activations, [row][64] x 16-bit, K contiguous as in memory; the 16-byte
//    chunk index is XOR-ed with (row & 7) ^ ((row >> 3) & 1) so that 16
//    consecutive rows read at one chunk hit distinct banks. A fragment is one
//    16-byte read per lane.
//  * weights, [k][256] x 16-bit, N contiguous as in memory (a straight copy
//    of 16-byte runs), rows padded to 576 bytes. The MFMA wants 8 K-values of
//    one column per lane: gfx950's transposing LDS read (ds_read_b64_tr_b16)
//    gives each lane of a 16-lane group 4 K-values of its column from a 4 x 16
//    block, so a fragment is two such reads. With the 576-byte stride, the 32
//    lanes of a half-wave read 32 distinct 8-byte bank slots.
//
// The expert and row range of a workgroup come from the device-resident
// offsets (see find_tile_rows), so the grid is sized from the row capacity
// and needs no host synchronisation; surplus workgroups exit at once.
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
constexpr int BM = 128;                  // rows per workgroup
constexpr int BK = 64;                   // K per step
constexpr int BNB = 256;                 // product columns per workgroup
constexpr int kBStride = BNB * 2 + 64;   // bytes per weight row in LDS
constexpr int kTileA = BM * BK * 2;      // 16 KB
constexpr int kTileB = BK * kBStride;    // 36 KB
constexpr int kStage = kTileA + kTileB;

__device__ __forceinline__ int a_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row & 7) ^ ((row >> 3) & 1))) << 4);
}

__device__ __forceinline__ uint32_t f16_bits(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<_Float16>(f));  // round to nearest even
}

// Two bf16 values -> two fp16 values (round to nearest even).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  return f16_bits(__uint_as_float(v << 16)) | (f16_bits(__uint_as_float(v & 0xffff0000u)) << 16);
}

__device__ __forceinline__ uint32_t pack2(short lo, short hi) {
  return static_cast<uint16_t>(lo) | (static_cast<uint32_t>(static_cast<uint16_t>(hi)) << 16);
}

// GEMM 1: bf16 x bf16 -> SiLU(gate) * up -> fp16 H.
// GEMM 2: fp16 H x (bf16 -> fp16) W_down -> fp32 Y.
enum Mode { kGateUp = 0, kDown = 1 };

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void ffn_gemm_bf16(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int n_experts,
    int64_t cap_rows, const uint16_t* __restrict__ W, void* __restrict__ Cout, int K,
    int N_out) {
  constexpr bool GATED = MODE == kGateUp;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];
  __shared__ int s_tile[3];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  if (wave == 0) {
    TileRows tr = find_tile_rows(offsets, n_experts, cap_rows, blockIdx.x, BM);
    if (lane == 0) {
      s_tile[0] = tr.expert;
      s_tile[1] = tr.row_begin;
      s_tile[2] = tr.row_end;
    }
  }
  __syncthreads();
  const int expert = s_tile[0];
  if (expert < 0) return;
  const int row_begin = s_tile[1], row_end = s_tile[2];

  // Output columns of this workgroup.
  constexpr int BN_OUT = GATED ? BNB / 2 : BNB;
  const int n0 = blockIdx.y * BN_OUT;
  const int ldw = GATED ? 2 * N_out : N_out;
  const uint16_t* Wexp = W + static_cast<int64_t>(expert) * K * ldw;

  // ---- global load assignment ----
  // A: 4 x 16 B per thread: rows (tid>>3) + 32*i, chunk tid&7.
  const int a_chunk = tid & 7;
  const uint16_t* a_ptr[4];
  bool a_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row_begin + (tid >> 3) + 32 * i;
    a_ok[i] = r < row_end;
    a_ptr[i] = A + static_cast<int64_t>(a_ok[i] ? r : row_begin) * K + a_chunk * 8;
  }
  // B: 8 x 16 B per thread: K rows (tid>>5) + 8*i, tile columns (tid&31)*8 .. +7.
  const int b_chunk = tid & 31;
  const int b_row0 = tid >> 5;
  int bcol;
  bool b_ok;
  if (GATED) {
    const int c = (b_chunk & 15) * 8;
    b_ok = n0 + c < N_out;
    bcol = (b_chunk < 16 ? 0 : N_out) + n0 + c;
  } else {
    b_ok = n0 + b_chunk * 8 < N_out;
    bcol = n0 + b_chunk * 8;
  }
  const uint16_t* b_ptr = Wexp + static_cast<int64_t>(b_row0) * ldw + (b_ok ? bcol : 0);

  uint4 ra[4];
  uint4 rb[8];

  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = a_ok[i] ? *reinterpret_cast<const uint4*>(a_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb[i] = b_ok ? *reinterpret_cast<const uint4*>(b_ptr + static_cast<int64_t>(k0 + 8 * i) * ldw)
                   : make_uint4(0, 0, 0, 0);
  };

  auto store_lds = [&](int stage) {
    unsigned char* sa = smem + stage * kStage;
    unsigned char* sb = sa + kTileA;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(sa + a_off((tid >> 3) + 32 * i, a_chunk)) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 v = rb[i];
      if (MODE == kDown) {
        v.x = bf16x2_to_f16x2(v.x);
        v.y = bf16x2_to_f16x2(v.y);
        v.z = bf16x2_to_f16x2(v.z);
        v.w = bf16x2_to_f16x2(v.w);
      }
      *reinterpret_cast<uint4*>(sb + (b_row0 + 8 * i) * kBStride + b_chunk * 16) = v;
    }
  };

  // ---- compute assignment: wave (wm, wn) ----
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5;
  int a_row[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) a_row[mb] = wm * 64 + mb * 32 + (lane & 31);
  // Transposing reads: lane j of 16-lane group g reads 8 bytes of weight row
  // kbase + (j >> 2) at column ncol + 4 * (j & 3), where the group covers
  // columns [16 * (g & 1), +16) of a 32-column block and K-half g >> 1. Lane
  // j then holds 4 K-values of column ncol_base + j.
  const int grp = lane >> 4, j16 = lane & 15;
  int b_col[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int blk = GATED ? ((q < 2 ? 0 : 128) + wn * 64 + (q & 1) * 32) : (wn * 128 + q * 32);
    b_col[q] = blk + 16 * (grp & 1) + 4 * (j16 & 3);
  }
  const int b_krow = 8 * (grp >> 1) + (j16 >> 2);  // + 16*kk, + 4 for the second read

  f32x16 acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][q][r] = 0.f;

  auto load_frags = [&](int stage, int kk, uint4(&fa)[2], uint4(&fb)[4]) {
    const unsigned char* sa = smem + stage * kStage;
    const int chunk = kk * 2 + half;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      fa[mb] = *reinterpret_cast<const uint4*>(sa + a_off(a_row[mb], chunk));
    const lds_u8* sb = (const lds_u8*)smem + stage * kStage + kTileA;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int off = (16 * kk + b_krow) * kBStride + b_col[q] * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + off));
      const s16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + off + 4 * kBStride));
      fb[q] = make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]),
                         pack2(hi[2], hi[3]));
    }
  };

  auto mfma_step = [&](const uint4(&fa)[2], const uint4(&fb)[4]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (MODE == kGateUp)
          acc[mb][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, fa[mb]), __builtin_bit_cast(bf16x8, fb[q]), acc[mb][q],
              0, 0, 0);
        else
          acc[mb][q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8, fa[mb]), __builtin_bit_cast(f16x8, fb[q]), acc[mb][q],
              0, 0, 0);
      }
  };

  const int nk = K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    // Fragments of the next K-slice are read while the current one multiplies.
    uint4 fa0[2], fb0[4], fa1[2], fb1[4];
    load_frags(cur, 0, fa0, fb0);
    load_frags(cur, 1, fa1, fb1);
    mfma_step(fa0, fb0);
    load_frags(cur, 2, fa0, fb0);
    mfma_step(fa1, fb1);
    load_frags(cur, 3, fa1, fb1);
    mfma_step(fa0, fb0);
    mfma_step(fa1, fb1);
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  // Accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4 and
  // column l%32 of its 32x32 tile.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int q = 0; q < (GATED ? 2 : 4); ++q) {
      const int col = n0 + (GATED ? wn * 64 + q * 32 : wn * 128 + q * 32) + (lane & 31);
      if (col >= N_out) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_begin + wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < row_end) {
          const int64_t o = static_cast<int64_t>(row) * N_out + col;
          if (GATED) {
            const float g = acc[mb][q][r];
            const float u = acc[mb][q + 2][r];
            static_cast<uint16_t*>(Cout)[o] =
                static_cast<uint16_t>(f16_bits(g / (1.f + __expf(-g)) * u));
          } else {
            static_cast<float*>(Cout)[o] = acc[mb][q][r];
          }
        }
      }
    }
  }
}

int64_t m_tiles(int64_t cap_rows, const int32_t* offsets, int n_experts) {
  // Each expert's segment may end in a partial tile: at most one extra per expert.
  return (cap_rows + BM - 1) / BM + (offsets ? n_experts : 0);
}

}  // namespace

hipError_t launch_gate_up_bf16(int n_experts, int64_t cap_rows, int D, int inter,
                               const void* x_perm, const int32_t* offsets, const void* w_gate_up,
                               void* h, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(m_tiles(cap_rows, offsets, n_experts)),
               (inter + BNB / 2 - 1) / (BNB / 2));
  ffn_gemm_bf16<kGateUp><<<g, kThreads, 0, s>>>(static_cast<const uint16_t*>(x_perm), offsets,
                                                n_experts, cap_rows,
                                                static_cast<const uint16_t*>(w_gate_up), h, D,
                                                inter);
  return hipGetLastError();
}

hipError_t launch_down_bf16(int n_experts, int64_t cap_rows, int D, int inter, const void* h,
                            const int32_t* offsets, const void* w_down, void* y, hipStream_t s) {
  const dim3 g(static_cast<unsigned>(m_tiles(cap_rows, offsets, n_experts)), (D + BNB - 1) / BNB);
  ffn_gemm_bf16<kDown><<<g, kThreads, 0, s>>>(static_cast<const uint16_t*>(h), offsets,
                                              n_experts, cap_rows,
                                              static_cast<const uint16_t*>(w_down), y, inter, D);
  return hipGetLastError();
}

}  // namespace moe
