// Device-side split schedule shared by the INT2 decode path and the bf16
// baseline.
#pragma once

#include "oscar_device.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

// Split schedule of one decode call, computed by the 256 threads of one
// workgroup from the device-resident lengths: the pages of each request's
// L - skip_tokens paged tokens (the INT2 history skips the 320 bf16 sink and
// recent tokens; the all-bf16 baseline skips none).  The pages per split q
// is the smallest q >= max(kMinSplitPages, ceil(longest / kMaxSplits)) for
// which the batch needs at most `target` splits (request b taking
// S_b = ceil(pages_b / q)), found by bisection; when even one split per
// request exceeds the target, q is the longest request.  Each request's splits are equal (the last one shorter),
// numbered by a block-wide prefix scan.  Writes sched = {n_splits, then
// (request, page0, page1) per split} and req[b] = {first split, S_b}.
// n_splits <= max(target, B).
// Block-wide (256 threads) sum and max of an int: wave reduction, then the
// four wave results through LDS (red holds at least 4 ints).
__device__ __forceinline__ int block_sum(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ int block_max(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return max(max(red[0], red[1]), max(red[2], red[3]));
}

__device__ void schedule_splits(const int32_t* __restrict__ seq_lens, int batch, int skip_tokens, int target,
                                int32_t* __restrict__ sched, int32_t* __restrict__ req) {
  const int tid = threadIdx.x;
  constexpr int kCached = 1024;   // history page counts kept in LDS (the rest re-read)
  __shared__ int red[4];
  __shared__ int scan[256];
  __shared__ int s_off;
  __shared__ int pages_s[kCached];
  auto pages_from_len = [&](int b) {
    const int n_hist = max(0, seq_lens[b] - skip_tokens);
    return (n_hist + kPage - 1) / kPage;
  };
  int local_max = 0, local_total = 0, local_busy = 0;
  for (int b = tid; b < batch; b += 256) {
    const int pg = pages_from_len(b);
    if (b < kCached) pages_s[b] = pg;
    local_max = max(local_max, pg);
    local_total += pg;
    local_busy += pg > 0;
  }
  auto pages_of = [&](int b) { return b < kCached ? pages_s[b] : pages_from_len(b); };
  const int max_pages = block_max(local_max, red);
  const int total = block_sum(local_total, red);
  const int busy = block_sum(local_busy, red);   // requests with history
  // bracket: count(q) >= total / q needs q >= total / target, and
  // count(q) <= total / q + busy holds at q = total / (target - busy)
  int lo = max(max(kMinSplitPages, (max_pages + kMaxSplits - 1) / kMaxSplits),   // <= kMaxSplits per request
               (total + target - 1) / target);
  int hi = target > busy ? (total + target - busy - 1) / (target - busy) : max_pages;
  hi = max(lo, min(hi, max_pages));
  while (lo < hi) {   // uniform across the block
    const int mid = (lo + hi) / 2;
    int local = 0;
    for (int b = tid; b < batch; b += 256) local += (pages_of(b) + mid - 1) / mid;
    if (block_sum(local, red) <= target) hi = mid;
    else lo = mid + 1;
  }
  const int q = lo;
  if (tid == 0) s_off = 0;
  __syncthreads();
  for (int base = 0; base < batch; base += 256) {
    const int b = base + tid;
    int pages = 0, nsp = 0;
    if (b < batch) {
      pages = pages_of(b);
      nsp = (pages + q - 1) / q;
    }
    scan[tid] = nsp;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int first = s_off + scan[tid] - nsp;
    if (b < batch) {
      req[2 * b] = first;
      req[2 * b + 1] = nsp;
      const int per = nsp > 0 ? (pages + nsp - 1) / nsp : 0;
      for (int i = 0; i < nsp; ++i) {
        int32_t* e = sched + 1 + 3 * (first + i);
        e[0] = b;
        e[1] = i * per;
        e[2] = min((i + 1) * per, pages);
      }
    }
    __syncthreads();
    if (tid == 0) s_off += scan[255];
    __syncthreads();
  }
  if (tid == 0) sched[0] = s_off;
}

}  // namespace
}  // namespace oscar
