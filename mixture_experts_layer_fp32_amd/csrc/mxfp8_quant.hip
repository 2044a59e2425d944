// MXFP8 quantization for the MXFP8 expert FFN: activation rows and packed
// weights.
//
// The pages name an MXFP8 transform of the MoE layer (torchtitan issue 5554)
// without defining it; the format is the OCP Microscaling (MX) v1.0 MXFP8:
// E4M3 elements (bias 7, no infinities, largest magnitude 448) in blocks of 32
// consecutive values along the contraction dimension, each block sharing an
// E8M0 scale 2^s with s = floor(log2(amax)) - 8 clamped to [-127, 127]
// (all-zero block: s = -127). Elements are v / 2^s rounded to the nearest
// E4M3 value, ties to even, saturating at 448.
//
// Arithmetic: v / 2^s is a multiplication by an exact power of two (2^-s is a
// normal fp32 for every s a bf16 block can produce), so it is exact except
// where the quotient falls below fp32's normal range, far below E4M3's
// smallest subnormal (2^-9), where it rounds to zero either way. The E4M3
// rounding then works on the fp32 bits.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Block exponent s for a block maximum magnitude amax (fp32 bits, sign clear).
__device__ __forceinline__ int mx_block_exp(uint32_t amax_bits) {
  const int ef = static_cast<int>(amax_bits >> 23);  // biased exponent; 0 for zero/subnormal
  return ef == 0 ? -127 : max(ef - 127 - 8, -127);
}

// fp32 y (already divided by the block scale, |y| < 512) -> E4M3 code.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x3C800000u) {  // |y| >= 2^-6: normal E4M3
    // Rebias the exponent (fp32 bias 127 -> E4M3 bias 7) and round the
    // 23-bit mantissa to 3 bits, ties to even; a carry moves into the exponent.
    const uint32_t t = a - (120u << 23);
    const uint32_t r = (t + 0x7FFFFu + ((t >> 20) & 1u)) >> 20;
    code = min(r, 0x7Eu);  // saturate at 448 (0x7F would be NaN)
  } else {
    // Subnormal range: multiples of 2^-9 (rounding up to 8 gives code 8, the
    // smallest normal). |y| * 512 is exact; rint rounds ties to even.
    code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.f));
  }
  return sign | code;
}

__device__ __forceinline__ float scale_down(float v, int s) {
  return v * __uint_as_float(static_cast<uint32_t>(127 - s) << 23);  // v * 2^-s
}

// Activation rows [rows][K] bf16 -> codes [rows][K], scales [rows][K/32].
// A thread takes 8 consecutive values; the 4 threads of a DPP quad hold one
// 32-value block.
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(
    const uint4* __restrict__ x, int64_t n_vec, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const bool live = g < n_vec;  // n_vec = rows * K / 8, a multiple of 4
  uint4 v = live ? x[g] : make_uint4(0, 0, 0, 0);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = max(amax, __float_as_uint(f[i]) & 0x7fffffffu);
  // Quad maximum (lanes 4q .. 4q + 3): exchange with lane ^ 1, then lane ^ 2.
  amax = max(amax, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(amax), 0xB1, 0xF, 0xF, false)));
  amax = max(amax, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(amax), 0x4E, 0xF, 0xF, false)));
  const int s = mx_block_exp(amax);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= e4m3_code(scale_down(f[i], s)) << (8 * i);
    hi |= e4m3_code(scale_down(f[4 + i], s)) << (8 * i);
  }
  if (live) {
    codes[g] = make_uint2(lo, hi);
    if ((threadIdx.x & 3) == 0) scales[g >> 2] = static_cast<uint8_t>(s + 127);
  }
}

// Weights [n][K][N] bf16 -> codes [n][N][K], scales [n][N][K/32]: each output
// column is quantized along K. A workgroup stages a 32 x 256 tile of one
// expert in LDS; thread j takes column n0 + j and writes its 32 codes.
__global__ __launch_bounds__(kThreads) void pack_weights_kernel(
    const uint16_t* __restrict__ w, int K, int N, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  __shared__ uint16_t tile[32][kThreads];
  const int k0 = blockIdx.x * 32, n0 = blockIdx.y * kThreads, e = blockIdx.z;
  const int j = threadIdx.x;
  const uint16_t* we = w + static_cast<int64_t>(e) * K * N;
  for (int r = 0; r < 32; ++r)
    tile[r][j] = n0 + j < N ? we[static_cast<int64_t>(k0 + r) * N + n0 + j] : uint16_t(0);
  __syncthreads();
  if (n0 + j >= N) return;
  float f[32];
  uint32_t amax = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    f[r] = __uint_as_float(static_cast<uint32_t>(tile[r][j]) << 16);
    amax = max(amax, __float_as_uint(f[r]) & 0x7fffffffu);
  }
  const int s = mx_block_exp(amax);
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    q[i] = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) q[i] |= e4m3_code(scale_down(f[4 * i + b], s)) << (8 * b);
  }
  const int64_t col = static_cast<int64_t>(e) * N + n0 + j;
  uint4* dst = reinterpret_cast<uint4*>(codes + col * K + k0);
  dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
  dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
  scales[col * (K / 32) + blockIdx.x] = static_cast<uint8_t>(s + 127);
}

}  // namespace

hipError_t launch_mx_quantize_rows(int64_t rows, int K, const void* x, void* codes, void* scales,
                                   hipStream_t s) {
  const int64_t n_vec = rows * K / 8;
  if (n_vec == 0) return hipSuccess;
  const int64_t grid = (n_vec + kThreads - 1) / kThreads;
  quantize_rows_kernel<<<static_cast<unsigned>(grid), kThreads, 0, s>>>(
      static_cast<const uint4*>(x), n_vec, static_cast<uint2*>(codes),
      static_cast<uint8_t*>(scales));
  return hipGetLastError();
}

hipError_t launch_mx_pack_weights(int n, int K, int N, const void* w, void* codes, void* scales,
                                  hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid(K / 32, (N + kThreads - 1) / kThreads, n);
  pack_weights_kernel<<<grid, kThreads, 0, s>>>(static_cast<const uint16_t*>(w), K, N,
                                                static_cast<uint8_t*>(codes),
                                                static_cast<uint8_t*>(scales));
  return hipGetLastError();
}

}  // namespace moe
