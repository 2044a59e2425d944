// Preprocess and permute: per-expert counts, offsets, split sizes, and an
// expert-contiguous copy of the (token, expert) pairs.
//
// Page "Expert Parallel (EP)", Communication Pattern: stage 1 computes the
// per-expert token counts and split sizes, stage 2 permutes tokens by expert
// assignment. Page "Worked Example", Step 2: every chosen expert gives the
// token one dispatch entry.
//
// The row order is fixed (expert-major, then ascending token), so the result
// does not depend on the order atomics happen to run in:
//   1. count:  per block of PB tokens, LDS integer atomics count the pairs of
//              each in-range expert (a count does not depend on order); for
//              few pairs the scan's workgroup counts them itself (one launch
//              fewer).
//   2. scan:   one workgroup turns the block counts into per-expert totals,
//              exclusive offsets, each block's first row per expert, and the
//              split sizes per owning rank.
//   3. rank + copy: per block, every wavefront ORs its lanes' bits into one
//              64-bit mask per expert in LDS; a pair's row is the block's
//              first row for the expert plus the popcount of the masks of
//              earlier wavefronts and of lower lanes: ascending token order.
//              Each block is served by S workgroups that all build its masks
//              (a few KB of indices) and each write the rows, positions and
//              copies of their own 1/S of its tokens: one wavefront per token
//              reads its row once (16-byte vectors) and writes it to each of
//              its in-range rows.
#include <algorithm>

#include "moe_internal.h"

namespace moe {

int perm_token_block(int T, int n) {
  // Keep block count x experts within the scan's LDS (48 KB of ints).
  int pb = kPermBlock;
  while (static_cast<int64_t>((T + pb - 1) / pb) * n > kPermMaxBlockCounts) pb *= 2;
  return pb;
}

namespace {

constexpr int kThreads = 256;
constexpr int kScanThreads = 1024;
// Pairs up to which the scan workgroup counts them itself: beyond a few per
// thread the LDS atomics of one CU cost more than the count kernel's launch.
constexpr int kScanCountPairs = 4 * kScanThreads;

// Exclusive prefix over the workgroup of one value per thread (NT threads);
// ws is LDS scratch of 2 NT / 64 + 1 ints. *total gets the sum of all values.
template <int NT>
__device__ int wg_exclusive_scan(int v, int* ws, int* total) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) ws[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int wt = lane < kWaves ? ws[lane] : 0;
    int wi = wt;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const int y = __shfl_up(wi, off, 64);
      if (lane >= off) wi += y;
    }
    if (lane < kWaves) ws[kWaves + lane] = wi - wt;
    if (lane == kWaves - 1) ws[2 * kWaves] = wi;
  }
  __syncthreads();
  *total = ws[2 * kWaves];
  return ws[kWaves + wave] + incl - v;
}

// Per-expert totals tot[n] (LDS) -> counts, offsets (n + 1) and, when split
// is given, the pairs per owning rank. tot[] is overwritten with the experts'
// first rows. ws: LDS scratch for wg_exclusive_scan<NT>.
template <int NT>
__device__ void write_offsets(int* tot, int* ws, int n, int e_begin, int e_per_rank,
                              int ep_size, int32_t* __restrict__ counts,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ split) {
  const int tid = threadIdx.x;
  // Each thread owns a contiguous run of experts.
  const int per = (n + NT - 1) / NT;
  const int j0 = tid * per;
  int local = 0;
  for (int j = j0; j < min(n, j0 + per); ++j) local += tot[j];
  int total;
  int run = wg_exclusive_scan<NT>(local, ws, &total);
  for (int j = j0; j < min(n, j0 + per); ++j) {
    const int c = tot[j];
    counts[j] = c;
    offsets[j] = run;
    tot[j] = run;  // now the expert's first row
    run += c;
  }
  if (tid == 0) offsets[n] = total;
  __syncthreads();
  if (split != nullptr) {
    // Rank q owns experts [q*e_per_rank, (q+1)*e_per_rank); sum the counts of
    // the in-range ones (first rows are monotone, so take a difference).
    for (int q = tid; q < ep_size; q += NT) {
      const int lo = max(q * e_per_rank - e_begin, 0);
      const int hi = min((q + 1) * e_per_rank - e_begin, n);
      split[q] = hi > lo ? (hi < n ? tot[hi] : total) - tot[lo] : 0;
    }
  }
}

__global__ __launch_bounds__(kThreads) void count_kernel(const int32_t* __restrict__ idx,
                                                         int T, int k, int e_begin, int n,
                                                         int pb, int32_t* __restrict__ block_counts) {
  extern __shared__ int cnt[];
  for (int j = threadIdx.x; j < n; j += kThreads) cnt[j] = 0;
  __syncthreads();
  const int t_begin = blockIdx.x * pb;
  const int t_end = min(T, t_begin + pb);
  for (int64_t i = static_cast<int64_t>(t_begin) * k + threadIdx.x;
       i < static_cast<int64_t>(t_end) * k; i += kThreads) {
    const int e = idx[i] - e_begin;
    if (e >= 0 && e < n) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += kThreads)
    block_counts[static_cast<int64_t>(blockIdx.x) * n + j] = cnt[j];
}

// The scan of one workgroup over the block counts: each block's first row per
// expert into block_base[nb][n], plus the totals. COUNT: the workgroup also
// counts the pairs itself (LDS integer atomics over idx; few pairs: one
// launch instead of two), else it reads the count kernel's block_counts.
template <bool COUNT>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t* __restrict__ block_counts, const int32_t* __restrict__ idx, int T, int k,
    int pb, int nb, int n, int e_begin, int e_per_rank, int ep_size,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ split,
    int32_t* __restrict__ block_base) {
  extern __shared__ int sm[];
  int* bc = sm;            // [nb][n]
  int* tot = bc + nb * n;  // [n]
  int* ws = tot + n;       // [2 * 16 + 1]
  const int tid = threadIdx.x;
  if (COUNT) {
    for (int i = tid; i < nb * n; i += kScanThreads) bc[i] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += kScanThreads) {
      int* row = bc + (t / pb) * n;
      for (int j = 0; j < k; ++j) {
        const int e = idx[static_cast<int64_t>(t) * k + j] - e_begin;
        if (e >= 0 && e < n) atomicAdd(&row[e], 1);
      }
    }
  } else {
    for (int i = tid; i < nb * n; i += kScanThreads) bc[i] = block_counts[i];
  }
  __syncthreads();
  // Per expert: running count over blocks (each block's first row, relative).
  for (int j = tid; j < n; j += kScanThreads) {
    int run = 0;
    for (int b = 0; b < nb; ++b) {
      const int c = bc[b * n + j];
      bc[b * n + j] = run;
      run += c;
    }
    tot[j] = run;
  }
  __syncthreads();
  write_offsets<kScanThreads>(tot, ws, n, e_begin, e_per_rank, ep_size, counts, offsets, split);
  for (int i = tid; i < nb * n; i += kScanThreads) block_base[i] = bc[i] + tot[i % n];
}

// Rank (and copy) of block blockIdx.x / S; this workgroup owns the block's
// tokens [s * tps, (s + 1) * tps), s = blockIdx.x % S.
__global__ __launch_bounds__(kThreads) void rank_copy_kernel(
    const int32_t* __restrict__ idx, int T, int k, int e_begin, int n, int pb, int S, int tps,
    const int32_t* __restrict__ block_base, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ pos, const uint4* __restrict__ x, int row_vec,
    uint4* __restrict__ x_perm) {
  extern __shared__ unsigned long long masks[];            // [4][n]
  int* run = reinterpret_cast<int*>(masks + 4 * n);         // [n]
  int* own_pos = run + n;                                   // [kThreads][k]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int blk = blockIdx.x / S, s = blockIdx.x - blk * S;
  const unsigned long long lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int t_block = blk * pb;
  const int own_lo = s * tps, own_hi = min(pb, own_lo + tps);
  for (int j = tid; j < n; j += kThreads)
    run[j] = block_base[static_cast<int64_t>(blk) * n + j];
  for (int sub = 0; sub < pb && sub < own_hi; sub += kThreads) {
    for (int j = tid; j < 4 * n; j += kThreads) masks[j] = 0ull;
    __syncthreads();
    const int u = sub + tid;  // token of the block
    const int t = t_block + u;
    const bool live = t < T && u < pb;
    if (live) {
      for (int j = 0; j < k; ++j) {
        const int e = idx[static_cast<int64_t>(t) * k + j] - e_begin;
        if (e >= 0 && e < n) atomicOr(&masks[wave * n + e], 1ull << lane);
      }
    }
    __syncthreads();
    if (live && u >= own_lo && u < own_hi) {
      for (int j = 0; j < k; ++j) {
        const int64_t q = static_cast<int64_t>(t) * k + j;
        const int e = idx[q] - e_begin;
        int r = -1;
        if (e >= 0 && e < n) {
          r = run[e];
#pragma unroll
          for (int w = 0; w < 3; ++w)
            if (w < wave) r += __popcll(masks[w * n + e]);
          r += __popcll(masks[wave * n + e] & lower);
          perm_src[r] = t;
        }
        pos[q] = r;
        own_pos[tid * k + j] = r;
      }
    }
    __syncthreads();
    if (x_perm != nullptr) {
      // One wavefront per owned token of this chunk. A token with no row in
      // [e_begin, e_end) (on the receive side of an EP rank, a third of the
      // tokens at top-8 of 256 experts over 8 ranks) is not read; two 16-byte
      // chunks of a row are in flight per lane.
      const int c_lo = max(own_lo, sub), c_hi = min(min(own_hi, sub + kThreads), T - t_block);
      for (int v = c_lo + wave; v < c_hi; v += kThreads / 64) {
        const int* pp = own_pos + (v - sub) * k;
        bool any = false;
        for (int j = 0; j < k; ++j) any |= pp[j] >= 0;
        if (!any) continue;  // (uniform: the wave's token)
        const uint4* src = x + static_cast<int64_t>(t_block + v) * row_vec;
#pragma unroll 2
        for (int c = lane; c < row_vec; c += 64) {
          const uint4 val = src[c];
          for (int j = 0; j < k; ++j) {
            const int r = pp[j];
            if (r >= 0) x_perm[static_cast<int64_t>(r) * row_vec + c] = val;
          }
        }
      }
    }
    for (int j = tid; j < n; j += kThreads)
      run[j] += __popcll(masks[j]) + __popcll(masks[n + j]) + __popcll(masks[2 * n + j]) +
                __popcll(masks[3 * n + j]);
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_permute(const moe_desc& d, const void* x, const int32_t* topk_idx,
                          int e_begin, int e_end, int32_t* counts, int32_t* offsets,
                          int32_t* split, int32_t* perm_src, int32_t* pos, void* x_perm,
                          int32_t* block_counts, int32_t* block_base, hipStream_t s) {
  const int n = e_end - e_begin;
  const int pb = perm_token_block(d.T, n);
  const int nb = (d.T + pb - 1) / pb;
  const size_t scan_lds = (static_cast<size_t>(nb) * n + n + 33) * sizeof(int);
  // Up to kScanCountPairs (token, expert) pairs the scan workgroup counts them
  // itself.
  if (static_cast<int64_t>(d.T) * d.top_k <= kScanCountPairs) {
    scan_kernel<true><<<1, kScanThreads, scan_lds, s>>>(
        nullptr, topk_idx, d.T, d.top_k, pb, nb, n, e_begin, d.E / d.ep_size, d.ep_size, counts,
        offsets, split, block_base);
  } else {
    count_kernel<<<nb, kThreads, n * sizeof(int), s>>>(topk_idx, d.T, d.top_k, e_begin, n, pb,
                                                      block_counts);
    scan_kernel<false><<<1, kScanThreads, scan_lds, s>>>(
        block_counts, nullptr, d.T, d.top_k, pb, nb, n, e_begin, d.E / d.ep_size, d.ep_size,
        counts, offsets, split, block_base);
  }
  if (nb == 0) return hipGetLastError();  // no tokens: zero counts, offsets and splits
  // Workgroups per block: about 4096 in all when the rows are copied (at least
  // 4 tokens each; every workgroup of a block redoes the block's LDS masks,
  // a small part of its work), one per block otherwise. Measured against 512
  // (with the copy loop above): rank-share receive side (32768 tokens of
  // 14 KB) 293 -> 190 us, skewed 128-expert layer 148 -> 144 us,
  // Mixtral-style within 1 us; 2048 gave 203 us, 8192 186 us.
  const int S = x_perm != nullptr ? std::max(1, std::min(pb / 4, (4096 + nb - 1) / nb)) : 1;
  const int tps = (pb + S - 1) / S;
  const size_t rank_lds = 4 * n * sizeof(unsigned long long) + n * sizeof(int) +
                          static_cast<size_t>(kThreads) * d.top_k * sizeof(int);
  const int elem = d.act_dtype == MOE_BF16 ? 2 : 4;
  rank_copy_kernel<<<nb * S, kThreads, rank_lds, s>>>(
      topk_idx, d.T, d.top_k, e_begin, n, pb, S, tps, block_base, perm_src, pos,
      static_cast<const uint4*>(x), d.D * elem / 16, static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
