// All-bf16 KV-cache decode attention: the baseline the INT2 path is measured
// against (page "Together AI 开源 OSCAR…", section "结果", and page
// "超越TurboQuant…", section "OSCAR的另一个关键点是", compare OSCAR with a
// BF16 KV cache).  Every one of a request's L tokens sits in bf16 pages;
// nothing is rotated or quantized.  It is built to run at HBM speed, so the
// INT2 / BF16 step ratio compares two bandwidth-bound kernels.
//
// Page block of one (page, KV head): keys [64][128] then values [64][128],
// bf16, 32 KB.  Decode is split-K over pages with the same device-side split
// schedule as the INT2 path (no tokens skipped), one 64-lane wave per
// (split, KV head):
//   * q.k: lane = token, reading its 256-byte key row in sixteen 16-byte
//     loads; the query heads' rows come from LDS;
//   * p.v: lane = (8-channel group, token residue mod 4), sixteen 16-byte
//     loads coalesced along value rows, reduced over the residues at the end;
//   * each wave loads a whole page (32 KB) and then computes on it; two
//     waves per SIMD overlap one's loads with the other's arithmetic (loading
//     the next page during the arithmetic needs more registers than two
//     waves per SIMD allow).
// A separate merge combines the splits per (request, query head).
#include <hip/hip_ext.h>
#include <math.h>

#include "schedule.h"

namespace oscar {
namespace {

constexpr int kBlockElems = 2 * kPage * kDim;   // bf16 elements per (page, KV head) block

struct BaseParams {
  const uint16_t* pages;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const uint16_t* q;
  const int32_t* sched;
  float* po;          // [slots][Hq][128]
  float* plse;        // [slots][Hq]
  int32_t max_pages;
  int32_t hkv;
  int32_t hq;
};

__global__ void __launch_bounds__(256)
base_schedule_kernel(const int32_t* __restrict__ seq_lens, int batch, int target, int32_t* __restrict__ sched,
                     int32_t* __restrict__ req) {
  schedule_splits(seq_lens, batch, 0, target, sched, req);
}

__device__ __forceinline__ void lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int GQ>
__global__ void __launch_bounds__(64) base_hist_kernel(BaseParams a) {
  const int split = blockIdx.x, kvh = blockIdx.y;
  if (split >= a.sched[0]) return;   // unused slot (uniform)
  const int b = a.sched[1 + 3 * split];
  const int p0 = a.sched[2 + 3 * split];
  const int p1 = a.sched[3 + 3 * split];
  const int lane = threadIdx.x, cg = lane & 15, res = lane >> 4;
  const int L = a.seq_lens[b];
  __shared__ float qs[GQ][kDim];
  __shared__ float ps[GQ][kPage];
  const size_t head0 = static_cast<size_t>(b) * a.hq + static_cast<size_t>(kvh) * GQ;
  for (int i = lane; i < GQ * kDim; i += 64)
    qs[i / kDim][i % kDim] = bf16_to_f32(a.q[head0 * kDim + i]) * kScoreScaleLog2;
  lds_fence();
  const int32_t* pt = a.page_table + static_cast<size_t>(b) * a.max_pages;
  auto block = [&](int p) {
    return a.pages + (static_cast<size_t>(pt[p]) * a.hkv + kvh) * kBlockElems;
  };
  uint4 krow[kDim / 8], vrow[16];
  auto load_k = [&](int p) {
    const uint4* row = reinterpret_cast<const uint4*>(block(p) + lane * kDim);   // rows past L are read, masked
#pragma unroll
    for (int v8 = 0; v8 < kDim / 8; ++v8) krow[v8] = row[v8];
  };
  // value rows are read whole by each load (16 lanes per 256-byte row) and
  // once per page: non-temporal, as in the INT2 kernel.  The key loads stay
  // ordinary: a lane reads its own token's row, so each cache line serves
  // eight consecutive loads (non-temporal key loads doubled the traffic).
  auto load_v = [&](int p) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const uint16_t* vb = block(p) + kPage * kDim;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const v4u w = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(vb + (res + 4 * i) * kDim + 8 * cg));
      vrow[i] = make_uint4(w.x, w.y, w.z, w.w);
    }
  };
  float m[GQ], l[GQ], acc[GQ][8];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
#pragma unroll 1
  for (int p = p0; p < p1; ++p) {
    // the query rows are re-read from LDS every page (broadcast reads)
    // instead of being held in 128 x GQ registers
    __asm__ volatile("" ::: "memory");
    load_k(p);
    load_v(p);
    const int n_valid = min(kPage, L - p * kPage);
    // ---- scores, lane = token
    float sc[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) sc[h] = 0.f;
#pragma unroll
    for (int v8 = 0; v8 < kDim / 8; ++v8) {
      // keep each 8-channel step's query reads next to their use
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t ws[4] = {krow[v8].x, krow[v8].y, krow[v8].z, krow[v8].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(ws[j] << 16);
        const float hi = __uint_as_float(ws[j] & 0xFFFF0000u);
        const int ch = v8 * 8 + 2 * j;
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
          sc[h] = __builtin_fmaf(qs[h][ch], lo, sc[h]);
          sc[h] = __builtin_fmaf(qs[h][ch + 1], hi, sc[h]);
        }
      }
    }
    // ---- online softmax per head (base-2 units)
    const bool valid = lane < n_valid;
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const float s = valid ? sc[h] : -INFINITY;
      const float mn = fmaxf(m[h], wave_max(s));
      const float alpha = m[h] == -INFINITY ? 0.f : exp2f(m[h] - mn);
      const float pr = valid ? exp2f(s - mn) : 0.f;
      l[h] = l[h] * alpha + wave_sum(pr);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      m[h] = mn;
      ps[h][lane] = pr;
    }
    lds_fence();
    // ---- p . v, lane = (channel group cg, token residue res)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = res + 4 * i;
      const uint32_t ws[4] = {vrow[i].x, vrow[i].y, vrow[i].z, vrow[i].w};
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float pt_ = ps[h][t];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[h][2 * j] = __builtin_fmaf(pt_, __uint_as_float(ws[j] << 16), acc[h][2 * j]);
          acc[h][2 * j + 1] = __builtin_fmaf(pt_, __uint_as_float(ws[j] & 0xFFFF0000u), acc[h][2 * j + 1]);
        }
      }
    }
    lds_fence();   // ps is rewritten by the next page
  }
  // ---- partial output of this split
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const size_t pidx = static_cast<size_t>(split) * a.hq + static_cast<size_t>(kvh) * GQ + h;
    const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (res == 0) a.po[pidx * kDim + 8 * cg + e] = v * inv;
    }
    if (lane == 0) a.plse[pidx] = l[h] > 0.f ? (m[h] + log2f(l[h])) * kLn2 : -INFINITY;
  }
}

struct BaseMergeParams {
  const float* ho;
  const float* hlse;
  const int32_t* req;
  float* out;
  float* lse_out;
  int32_t hq;
};

// Workgroup = (query head, request), 256 threads: thread t weighs split t,
// both halves of the workgroup sum alternate splits.
__global__ void __launch_bounds__(256) base_merge_kernel(BaseMergeParams a) {
  const int head = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ float red[4];
  __shared__ float w[kMaxSplits + 1];
  __shared__ float part[2][kDim];
  const int first = a.req[2 * b], count = a.req[2 * b + 1];
  const float lv = tid < count ? a.hlse[static_cast<size_t>(first + tid) * a.hq + head] : -INFINITY;
  float mx = wave_max(lv);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float e = tid < count && mx != -INFINITY ? expf(lv - mx) : 0.f;
  float den = wave_sum(e);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = den;
  __syncthreads();
  den = (red[0] + red[1]) + (red[2] + red[3]);
  if (tid < count) w[tid] = den > 0.f ? e / den : 0.f;
  __syncthreads();
  const int k = tid & (kDim - 1), par = tid >> 7;
  const float* hp = a.ho + (static_cast<size_t>(first) * a.hq + head) * kDim + k;
  const size_t stride = static_cast<size_t>(a.hq) * kDim;
  float acc = 0.f;
  for (int sp = par; sp < count; sp += 2) acc = __builtin_fmaf(w[sp], hp[static_cast<size_t>(sp) * stride], acc);
  part[par][k] = acc;
  __syncthreads();
  const size_t bh = static_cast<size_t>(b) * a.hq + head;
  if (tid < kDim) a.out[bh * kDim + tid] = part[0][tid] + part[1][tid];
  if (a.lse_out != nullptr && tid == 0) a.lse_out[bh] = den > 0.f ? mx + logf(den) : -INFINITY;
}

// Copy tokens [pos_begin, pos_begin + n) of one request into its pages:
// workgroup = 16 tokens of one KV head, K or V; thread = 16 bytes of a row.
__global__ void __launch_bounds__(256)
base_fill_kernel(uint16_t* __restrict__ pages, const int32_t* __restrict__ page_table, int max_pages, int hkv,
                 int request, int pos_begin, int n_tokens, const uint16_t* __restrict__ k_tokens,
                 const uint16_t* __restrict__ v_tokens) {
  const int kvh = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4), piece = threadIdx.x & 15;
  if (t >= n_tokens) return;
  const int pos = pos_begin + t;
  const int phys = page_table[static_cast<size_t>(request) * max_pages + pos / kPage];
  const uint16_t* src = (is_v ? v_tokens : k_tokens) + (static_cast<size_t>(t) * hkv + kvh) * kDim;
  uint16_t* dst = pages + (static_cast<size_t>(phys) * hkv + kvh) * kBlockElems + (is_v ? kPage * kDim : 0) +
                  (pos % kPage) * kDim;
  reinterpret_cast<uint4*>(dst)[piece] = reinterpret_cast<const uint4*>(src)[piece];
}

// One decode step's append: token L_b - 1 of every request (seq_lens
// already count it).  Workgroup = (KV head, request), 32 threads: K then V.
__global__ void __launch_bounds__(32)
base_append_kernel(uint16_t* __restrict__ pages, const int32_t* __restrict__ page_table, int max_pages, int hkv,
                   const int32_t* __restrict__ seq_lens, const uint16_t* __restrict__ k_new,
                   const uint16_t* __restrict__ v_new) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int L = seq_lens[b];
  if (L < 1) return;
  const int pos = L - 1;
  const int phys = page_table[static_cast<size_t>(b) * max_pages + pos / kPage];
  const bool is_v = threadIdx.x >= 16;
  const int piece = threadIdx.x & 15;
  const uint16_t* src = (is_v ? v_new : k_new) + (static_cast<size_t>(b) * hkv + kvh) * kDim;
  uint16_t* dst = pages + (static_cast<size_t>(phys) * hkv + kvh) * kBlockElems + (is_v ? kPage * kDim : 0) +
                  (pos % kPage) * kDim;
  reinterpret_cast<uint4*>(dst)[piece] = reinterpret_cast<const uint4*>(src)[piece];
}

template <int GQ>
struct BaseHistRun {
  static hipError_t run(const BaseParams& p, int slots, int hkv, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    const dim3 grid(slots, hkv);
    if (ev0 != nullptr && ev1 != nullptr)
      hipExtLaunchKernelGGL(base_hist_kernel<GQ>, grid, dim3(64), 0, s, ev0, ev1, 0, p);
    else
      base_hist_kernel<GQ><<<grid, 64, 0, s>>>(p);
    return hipGetLastError();
  }
};

template <template <int> class F, typename... Args>
hipError_t dispatch_gq_base(int gq, Args... args) {
  switch (gq) {
    case 1: return F<1>::run(args...);
    case 2: return F<2>::run(args...);
    case 3: return F<3>::run(args...);
    case 4: return F<4>::run(args...);
    case 5: return F<5>::run(args...);
    case 6: return F<6>::run(args...);
    case 7: return F<7>::run(args...);
    default: return F<8>::run(args...);
  }
}

}  // namespace

BaseLayout base_layout(const oscar_dims& d, int32_t batch, int target_wg) {
  BaseLayout w;
  if (target_wg == 0) target_wg = d.num_q_heads / d.num_kv_heads > 4 ? kDefaultTargetWg / 2 : kDefaultTargetWg;
  w.target = (target_wg + d.num_kv_heads - 1) / d.num_kv_heads;
  w.slots = w.target + batch;
  const size_t cap = static_cast<size_t>((kMaxTargetWg + d.num_kv_heads - 1) / d.num_kv_heads) + batch;
  auto align256 = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t off = 0;
  w.off_sched = off;
  off = align256(off + (1 + 3 * cap) * sizeof(int32_t));
  w.off_req = off;
  off = align256(off + 2 * static_cast<size_t>(batch) * sizeof(int32_t));
  w.off_ho = off;
  off = align256(off + cap * d.num_q_heads * kDim * sizeof(float));
  w.off_hlse = off;
  off = align256(off + cap * d.num_q_heads * sizeof(float));
  w.total = off;
  return w;
}

hipError_t launch_base_decode(const oscar_dims& d, const oscar_bf16_cache& c, const uint16_t* q, uint8_t* ws,
                              const BaseLayout& lay, float* out, float* lse_out, hipStream_t s, hipEvent_t ev0,
                              hipEvent_t ev1) {
  int32_t* sched = reinterpret_cast<int32_t*>(ws + lay.off_sched);
  int32_t* req = reinterpret_cast<int32_t*>(ws + lay.off_req);
  base_schedule_kernel<<<1, 256, 0, s>>>(c.seq_lens, c.batch, lay.target, sched, req);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  BaseParams p;
  p.pages = c.pages;
  p.page_table = c.page_table;
  p.seq_lens = c.seq_lens;
  p.q = q;
  p.sched = sched;
  p.po = reinterpret_cast<float*>(ws + lay.off_ho);
  p.plse = reinterpret_cast<float*>(ws + lay.off_hlse);
  p.max_pages = c.max_pages_per_req;
  p.hkv = d.num_kv_heads;
  p.hq = d.num_q_heads;
  e = dispatch_gq_base<BaseHistRun>(d.num_q_heads / d.num_kv_heads, p, lay.slots, d.num_kv_heads, s, ev0, ev1);
  if (e != hipSuccess) return e;
  BaseMergeParams m;
  m.ho = p.po;
  m.hlse = p.plse;
  m.req = req;
  m.out = out;
  m.lse_out = lse_out;
  m.hq = d.num_q_heads;
  base_merge_kernel<<<dim3(d.num_q_heads, c.batch), 256, 0, s>>>(m);
  return hipGetLastError();
}

hipError_t launch_base_fill(const oscar_dims& d, const oscar_bf16_cache& c, int32_t request, int32_t pos_begin,
                            int32_t n_tokens, const uint16_t* k_tokens, const uint16_t* v_tokens, hipStream_t s) {
  const dim3 grid((n_tokens + 15) / 16, d.num_kv_heads, 2);
  base_fill_kernel<<<grid, 256, 0, s>>>(c.pages, c.page_table, c.max_pages_per_req, d.num_kv_heads, request,
                                        pos_begin, n_tokens, k_tokens, v_tokens);
  return hipGetLastError();
}

hipError_t launch_base_append(const oscar_dims& d, const oscar_bf16_cache& c, const uint16_t* k_new,
                              const uint16_t* v_new, hipStream_t s) {
  base_append_kernel<<<dim3(d.num_kv_heads, c.batch), 32, 0, s>>>(c.pages, c.page_table, c.max_pages_per_req,
                                                                   d.num_kv_heads, c.seq_lens, k_new, v_new);
  return hipGetLastError();
}

}  // namespace oscar
