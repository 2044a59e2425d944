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
//              each in-range expert (a count does not depend on order).
//   2. scan:   one workgroup turns the block counts into per-expert totals,
//              exclusive offsets, each block's first row per expert, and the
//              split sizes per owning rank.
//   3. rank:   per block, every wavefront ORs its lanes' bits into one 64-bit
//              mask per expert in LDS; a pair's row is the block's first row
//              for the expert plus the popcount of the masks of earlier
//              wavefronts and of lower lanes: ascending token order.
//   4. copy:   one wavefront per token reads its row once (16-byte vectors)
//              and writes it to each of its in-range rows.
#include "moe_internal.h"

namespace moe {

int perm_token_block(int T, int n) {
  // Keep block count x experts within the scan's LDS (12288 ints, 48 KB).
  int pb = kPermBlock;
  while (static_cast<int64_t>((T + pb - 1) / pb) * n > 12288) pb *= 2;
  return pb;
}

namespace {

constexpr int kThreads = 256;
constexpr int kScanThreads = 1024;

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

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t* __restrict__ block_counts, int nb, int n, int e_begin, int e_per_rank,
    int ep_size, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ split, int32_t* __restrict__ block_base) {
  extern __shared__ int sm[];
  int* bc = sm;            // [nb][n]
  int* tot = bc + nb * n;  // [n]
  int* scan = tot + n;     // [kScanThreads]
  const int tid = threadIdx.x;
  for (int i = tid; i < nb * n; i += kScanThreads) bc[i] = block_counts[i];
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
  // Exclusive scan of tot over experts: each thread owns a contiguous run.
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int j0 = tid * per;
  int local = 0;
  for (int j = j0; j < min(n, j0 + per); ++j) local += tot[j];
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int run = scan[tid] - local;  // exclusive prefix of this thread's run
  for (int j = j0; j < min(n, j0 + per); ++j) {
    const int c = tot[j];
    counts[j] = c;
    offsets[j] = run;
    tot[j] = run;  // now the expert's first row
    run += c;
  }
  if (tid == kScanThreads - 1) offsets[n] = scan[kScanThreads - 1];
  __syncthreads();
  for (int i = tid; i < nb * n; i += kScanThreads)
    block_base[i] = bc[i] + tot[i % n];
  if (split != nullptr) {
    // Rank q owns experts [q*e_per_rank, (q+1)*e_per_rank); sum the counts of
    // the in-range ones (first rows are monotone, so take a difference).
    for (int q = tid; q < ep_size; q += kScanThreads) {
      const int lo = max(q * e_per_rank - e_begin, 0);
      const int hi = min((q + 1) * e_per_rank - e_begin, n);
      split[q] = hi > lo ? (hi < n ? tot[hi] : scan[kScanThreads - 1]) - tot[lo] : 0;
    }
  }
}

__global__ __launch_bounds__(kThreads) void rank_kernel(const int32_t* __restrict__ idx, int T,
                                                        int k, int e_begin, int n, int pb,
                                                        const int32_t* __restrict__ block_base,
                                                        int32_t* __restrict__ perm_src,
                                                        int32_t* __restrict__ pos) {
  extern __shared__ unsigned long long masks[];            // [4][n]
  int* run = reinterpret_cast<int*>(masks + 4 * n);         // [n]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int j = tid; j < n; j += kThreads)
    run[j] = block_base[static_cast<int64_t>(blockIdx.x) * n + j];
  const unsigned long long lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int t_block = blockIdx.x * pb;
  for (int sub = 0; sub < pb; sub += kThreads) {
    for (int j = tid; j < 4 * n; j += kThreads) masks[j] = 0ull;
    __syncthreads();
    const int t = t_block + sub + tid;
    const bool live = t < T && sub + tid < pb;
    if (live) {
      for (int j = 0; j < k; ++j) {
        const int e = idx[static_cast<int64_t>(t) * k + j] - e_begin;
        if (e >= 0 && e < n) atomicOr(&masks[wave * n + e], 1ull << lane);
      }
    }
    __syncthreads();
    if (live) {
      for (int j = 0; j < k; ++j) {
        const int64_t q = static_cast<int64_t>(t) * k + j;
        const int e = idx[q] - e_begin;
        if (e >= 0 && e < n) {
          int r = run[e];
#pragma unroll
          for (int w = 0; w < 3; ++w)
            if (w < wave) r += __popcll(masks[w * n + e]);
          r += __popcll(masks[wave * n + e] & lower);
          pos[q] = r;
          perm_src[r] = t;
        } else {
          pos[q] = -1;
        }
      }
    }
    __syncthreads();
    for (int j = tid; j < n; j += kThreads)
      run[j] += __popcll(masks[j]) + __popcll(masks[n + j]) + __popcll(masks[2 * n + j]) +
                __popcll(masks[3 * n + j]);
    __syncthreads();
  }
}

// One wavefront per token: read the row once, write it to each in-range row.
__global__ __launch_bounds__(kThreads) void copy_rows_kernel(const uint4* __restrict__ x,
                                                             const int32_t* __restrict__ pos,
                                                             int T, int k, int row_vec,
                                                             uint4* __restrict__ x_perm) {
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  int p[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j)
    p[j] = j < k ? pos[static_cast<int64_t>(t) * k + j] : -1;
  const uint4* src = x + static_cast<int64_t>(t) * row_vec;
  for (int c = lane; c < row_vec; c += 64) {
    const uint4 v = src[c];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (p[j] >= 0) x_perm[static_cast<int64_t>(p[j]) * row_vec + c] = v;
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
  if (nb > 0)
    count_kernel<<<nb, kThreads, n * sizeof(int), s>>>(topk_idx, d.T, d.top_k, e_begin, n, pb,
                                                      block_counts);
  const size_t scan_lds = (static_cast<size_t>(nb) * n + n + kScanThreads) * sizeof(int);
  scan_kernel<<<1, kScanThreads, scan_lds, s>>>(block_counts, nb, n, e_begin,
                                               d.E / d.ep_size, d.ep_size, counts, offsets,
                                               split, block_base);
  if (nb == 0) return hipGetLastError();  // no tokens: zero counts, offsets and splits
  const size_t rank_lds = 4 * n * sizeof(unsigned long long) + n * sizeof(int);
  rank_kernel<<<nb, kThreads, rank_lds, s>>>(topk_idx, d.T, d.top_k, e_begin, n, pb,
                                            block_base, perm_src, pos);
  if (x_perm != nullptr) {
    const int elem = d.act_dtype == MOE_BF16 ? 2 : 4;
    const int row_vec = d.D * elem / 16;
    copy_rows_kernel<<<(d.T + 3) / 4, kThreads, 0, s>>>(
        static_cast<const uint4*>(x), pos, d.T, d.top_k, row_vec, static_cast<uint4*>(x_perm));
  }
  return hipGetLastError();
}

}  // namespace moe
