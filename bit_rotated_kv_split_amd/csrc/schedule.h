// Device-side split schedule shared by the INT2 decode path and the bf16
// baseline.
#pragma once

#include "oscar_device.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

// Split schedule of one decode call, computed by the first wave of a
// workgroup from the device-resident lengths: the pages of each request's
// L - skip_tokens paged tokens (the INT2 history skips the 320 bf16 sink and
// recent tokens; the all-bf16 baseline skips none).  The pages per split q
// is the smallest q >= max(kMinSplitPages, ceil(longest / kMaxSplits)) for
// which the batch needs at most `target` splits (request b taking
// S_b = ceil(pages_b / q)), found by bisection; when even one split per
// request exceeds the target, q is the longest request.  Each request's
// splits are equal (the last one shorter), numbered by a prefix scan over
// the requests.  Writes sched = {n_splits, then (request, page0, page1) per
// split} and req[b] = {first split, S_b}.  n_splits <= max(target, B).
//
// One wave does all of it with cross-lane operations and no workgroup
// barrier (the call sits on the critical path of every decode step); lanes
// 64 .. of the caller's workgroup return at once.  Lane l takes requests
// l, l + 64, ...; a request's split entries are written by its own lane, or,
// when it has more than kCoopSplits of them, by the whole wave.

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_scan_i(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    v += lane >= o ? t : 0;
  }
  return v;
}

constexpr int kCoopSplits = 64;

__device__ void schedule_splits(const int32_t* __restrict__ seq_lens, int batch, int skip_tokens, int target,
                                int32_t* __restrict__ sched, int32_t* __restrict__ req) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  constexpr int kCached = 1024;   // history page counts kept in LDS (the rest re-read)
  __shared__ int pages_s[kCached];
  auto pages_from_len = [&](int b) {
    const int n_hist = max(0, seq_lens[b] - skip_tokens);
    return (n_hist + kPage - 1) / kPage;
  };
  int local_max = 0, local_total = 0, local_busy = 0;
  for (int b = lane; b < batch; b += 64) {
    const int pg = pages_from_len(b);
    if (b < kCached) pages_s[b] = pg;
    local_max = max(local_max, pg);
    local_total += pg;
    local_busy += pg > 0;
  }
  // each lane reads back only the entries it wrote itself
  auto pages_of = [&](int b) { return b < kCached ? pages_s[b] : pages_from_len(b); };
  const int max_pages = wave_max_i(local_max);
  const int total = wave_sum_i(local_total);
  const int busy = wave_sum_i(local_busy);   // requests with history
  // bracket: count(q) >= total / q needs q >= total / target, and
  // count(q) <= total / q + busy holds at q = total / (target - busy)
  int lo = max(max(kMinSplitPages, (max_pages + kMaxSplits - 1) / kMaxSplits),   // <= kMaxSplits per request
               (total + target - 1) / target);
  int hi = target > busy ? (total + target - busy - 1) / (target - busy) : max_pages;
  hi = max(lo, min(hi, max_pages));
  while (lo < hi) {   // uniform across the wave
    const int mid = (lo + hi) / 2;
    int local = 0;
    for (int b = lane; b < batch; b += 64) local += (pages_of(b) + mid - 1) / mid;
    if (wave_sum_i(local) <= target) hi = mid;
    else lo = mid + 1;
  }
  const int q = lo;
  int off = 0;   // splits of the requests before this chunk (uniform)
  for (int base = 0; base < batch; base += 64) {
    const int b = base + lane;
    const int pages = b < batch ? pages_of(b) : 0;
    const int nsp = (pages + q - 1) / q;
    const int incl = wave_scan_i(nsp, lane);
    const int first = off + incl - nsp;
    const int per = nsp > 0 ? (pages + nsp - 1) / nsp : 0;
    if (b < batch) {
      req[2 * b] = first;
      req[2 * b + 1] = nsp;
    }
    if (nsp <= kCoopSplits) {
      for (int i = 0; i < nsp; ++i) {
        int32_t* e = sched + 1 + 3 * (first + i);
        e[0] = b;
        e[1] = i * per;
        e[2] = min((i + 1) * per, pages);
      }
    }
    // requests with many splits: one at a time, a split per lane
    uint64_t big = __ballot(nsp > kCoopSplits);
    while (big != 0) {
      const int src = __builtin_ctzll(big);
      big &= big - 1;
      const int rb = __shfl(b, src, 64), rfirst = __shfl(first, src, 64);
      const int rn = __shfl(nsp, src, 64), rper = __shfl(per, src, 64), rpages = __shfl(pages, src, 64);
      for (int i = lane; i < rn; i += 64) {
        int32_t* e = sched + 1 + 3 * (rfirst + i);
        e[0] = rb;
        e[1] = i * rper;
        e[2] = min((i + 1) * rper, rpages);
      }
    }
    off += __shfl(incl, 63, 64);
  }
  if (lane == 0) sched[0] = off;
}

}  // namespace
}  // namespace oscar
