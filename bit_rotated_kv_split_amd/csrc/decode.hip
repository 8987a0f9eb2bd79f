// Decode attention kernels over the three-region cache (page
// "超越TurboQuant：Together AI把2-bit KV Cache推向真实服务", section
// "OSCAR的另一个关键点是": an INT2 kernel over history, a bf16 kernel over
// sink and recent, and an online-softmax merge of the two).
//
//   qrot_kernel      q . R_K per (request, head), pre-scaled by log2(e)/sqrt(d),
//                    plus the per-group sums the zero-point term needs and
//                    the int8 digit operands of the matrix-core kernel.
//   hist_valu_kernel split-K over history pages on the vector ALU: lane =
//                    token for q.k, lane = channel pair for p.v.
//   bf16_kernel      sink + recent tokens with the unrotated query.
//   merge_kernel     LSE merge of the history splits, . R_V^T, merge with the
//                    bf16 partial.
//
// The factored score of a history token is
//   q_rot . k_hat = sum_groups ( scale * (q_rot . code) + zero * sum(q_rot) )
// and the value side accumulates (p * scale) * code plus (p * zero) per group,
// so dequantized values are never formed element by element.
#include <hip/hip_ext.h>
#include <math.h>

#include "decode_bf16.h"
#include "demote_device.h"
#include "schedule.h"

namespace oscar {
namespace {

// Fixed-point range of the matrix-core query operand: q * 2^26 / max|q|,
// held as four signed base-256 digits.  (Three digits, 2^22, saved one
// combine per score but moved a Lloyd-Max output by 2.3e-3 on the peaked
// edge-length test: rounding on the 1/64 slot grid left only 2^16 steps.)
constexpr float kQFixMax = 67108864.0f;

template <int GQ>
__global__ void __launch_bounds__(256)
qrot_kernel(const uint16_t* __restrict__ q, const float* __restrict__ r_k, int hq, int hkv, int G,
            float* __restrict__ qrot, float* __restrict__ qsum, uint8_t* __restrict__ qpack,
            const int32_t* __restrict__ seq_lens, int batch, int target, int32_t* __restrict__ sched,
            int32_t* __restrict__ req, float lm_ratio, DemoteStep dm) {
  // Row 0 of the grid (dispatched first) holds the split scheduler; rows
  // 1 .. B rotate the queries of request blockIdx.y - 1; the rows after
  // them, when launched, demote the step's oldest recent token, which
  // touches nothing the other rows read: rows B+1 .. 2B for request
  // blockIdx.y - B - 1 (threads 0..127 the key, 128..255 the value), or, for
  // small batches (3B+1 rows), rows B+1 .. 2B the key and 2B+1 .. 3B the
  // value, each by all 256 threads.
  const int kvh = blockIdx.x, b = static_cast<int>(blockIdx.y) - 1;
  if (b < 0) {
    if (kvh == 0) schedule_splits(seq_lens, batch, kBf16Tokens, target, sched, req);
    return;
  }
  if (b >= batch) {
    __shared__ QuantSmem<1> dsm[2];
    if (static_cast<int>(gridDim.y) > 1 + 2 * batch) {
      const bool is_v = b >= 2 * batch;
      demote_unit_g<256>(G, dm, kvh, b - (is_v ? 2 : 1) * batch, is_v, threadIdx.x, dsm[0]);
    } else {
      const int half = threadIdx.x >> 7;
      demote_unit_g(G, dm, kvh, b - batch, half != 0, threadIdx.x & 127, dsm[half]);
    }
    return;
  }
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int kRowGroups = 8, kGroupRows = kDim / kRowGroups;
  __shared__ float qs[GQ][kDim];
  __shared__ float part[kRowGroups][GQ][kDim];
  __shared__ float qr[GQ][kDim];
  __shared__ float qinv[GQ];
  const size_t head0 = static_cast<size_t>(b) * hq + static_cast<size_t>(kvh) * GQ;
  // q . R_K: thread (cq, rg) sums rows 16 rg .. 16 rg + 15 for channels
  // 4 cq .. 4 cq + 3 with 16-byte loads, requested together with the
  // queries, so the rows wait on memory once; the eight row-group partials
  // are added in LDS
  const int cq = tid & (kDim / 4 - 1), rg = tid >> 5;
  const float4* r4 = reinterpret_cast<const float4*>(r_k + static_cast<size_t>(kvh) * kDim * kDim);
  float4 rv[kGroupRows];
#pragma unroll
  for (int i = 0; i < kGroupRows; ++i) rv[i] = r4[(kGroupRows * rg + i) * (kDim / 4) + cq];
  for (int i = tid; i < GQ * kDim; i += 256) qs[i / kDim][i % kDim] = bf16_to_f32(q[head0 * kDim + i]);
  __syncthreads();
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kGroupRows; ++i) {
      const float x = qs[h][kGroupRows * rg + i];
      acc.x = __builtin_fmaf(x, rv[i].x, acc.x);
      acc.y = __builtin_fmaf(x, rv[i].y, acc.y);
      acc.z = __builtin_fmaf(x, rv[i].z, acc.z);
      acc.w = __builtin_fmaf(x, rv[i].w, acc.w);
    }
    *reinterpret_cast<float4*>(&part[rg][h][4 * cq]) = acc;
  }
  __syncthreads();
  for (int i = tid; i < GQ * kDim; i += 256) {
    const int h = i / kDim, c = i % kDim;
    float t = part[0][h][c];
#pragma unroll
    for (int g = 1; g < kRowGroups; ++g) t += part[g][h][c];
    const float v = t * kScoreScaleLog2;
    qr[h][c] = v;
    qrot[(head0 + h) * kDim + c] = v;
  }
  __syncthreads();
  // per-group sums and the largest magnitude, one wave per head
  for (int h = wave; h < GQ; h += 4) {
    const float v0 = qr[h][lane], v1 = qr[h][lane + 64];
    const float mx = wave_reduce_dpp(fmaxf(fabsf(v0), fabsf(v1)), WaveMax());
    if (lane == 0) qinv[h] = mx > 0.f ? kQFixMax / mx : 0.f;
    for (int gi = 0; gi < 4; ++gi) {
      const int lo = gi * G, hi = lo + G;
      float sgi = 0.f;
      if (lo < kDim) {   // uniform: groups past the head dimension hold 0
        sgi = (lane >= lo && lane < hi ? v0 : 0.f) + (lane + 64 >= lo && lane + 64 < hi ? v1 : 0.f);
        sgi = wave_reduce_dpp(sgi, WaveAdd());
      }
      if (lane == 0) qsum[(head0 + h) * 4 + gi] = sgi;
    }
    if (lane == 0) {
      float* sc = reinterpret_cast<float*>(qpack + (static_cast<size_t>(b) * hkv + kvh) * kQPackBytes +
                                           kQPackScaleOffset);
      sc[h] = mx > 0.f ? mx / kQFixMax : 0.f;
    }
  }
  __syncthreads();
  // int8 digit operands: row = 4*h + digit, 32 rows; for channel half hf and
  // lane group kg, byte e = 4*j + b2 of the row holds channel
  // 16*(4*hf + kg) + 4*b2 + j.  The matrix-core kernel feeds that channel's
  // 2-bit code masked in place, i.e. multiplied by 4^j (64 (code - 2) for
  // j = 3, whose codes are stored XOR 2), so the operand holds q / 4^j for
  // those slots (rounded on its own, coarser grid).
  uint8_t* qp = qpack + (static_cast<size_t>(b) * hkv + kvh) * kQPackBytes;
  // the second operand (Lloyd-Max codebook only) holds q * lm_ratio on the
  // same fixed-point grid, so both code planes accumulate into one result
  const int n_ops = lm_ratio != 0.f ? 2 : 1;
  for (int op = 0; op < n_ops; ++op) {
    uint32_t* qpw = reinterpret_cast<uint32_t*>(qp + op * kQPackOperandBytes);
    const float mul = op == 0 ? 1.f : lm_ratio;
    // thread (hf, kg, h, j) = tid: the four digit rows of head h for dword j
    // of channel half hf, lane group kg; each value is decomposed once and
    // its digits go to the four rows' words (word index
    // ((hf * 4 + kg) * kQPackRows + 4 h + digit) * 4 + j)
    static_assert(2 * 4 * (kQPackRows / 4) * 4 == 256, "one thread per four-row word group");
    {
      const int j = tid & 3, h = (tid >> 2) & (kQPackRows / 4 - 1), kg = (tid >> 5) & 3, hf = tid >> 7;
      uint32_t word[4] = {0u, 0u, 0u, 0u};
      if (h < GQ) {
        const float slot = j == 1 ? 0.25f : (j == 2 ? 0.0625f : (j == 3 ? 0.015625f : 1.f));
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) {
          const int ch = 16 * (4 * hf + kg) + 4 * b2 + j;
          const int qi = static_cast<int>(rintf(qr[h][ch] * mul * qinv[h] * slot));
          const int d0 = ((qi + 128) & 255) - 128;
          const int q1 = (qi - d0) >> 8;
          const int d1 = ((q1 + 128) & 255) - 128;
          const int q2 = (q1 - d1) >> 8;
          const int d2 = ((q2 + 128) & 255) - 128;
          const int d3 = (q2 - d2) >> 8;
          word[0] |= static_cast<uint32_t>(d0 & 255) << (8 * b2);
          word[1] |= static_cast<uint32_t>(d1 & 255) << (8 * b2);
          word[2] |= static_cast<uint32_t>(d2 & 255) << (8 * b2);
          word[3] |= static_cast<uint32_t>(d3 & 255) << (8 * b2);
        }
      }
      const int base = ((hf * 4 + kg) * kQPackRows + 4 * h) * 4 + j;
#pragma unroll
      for (int d = 0; d < 4; ++d) qpw[base + 4 * d] = word[d];
    }
  }
  if (tid >= GQ && tid < 8) {
    float* sc = reinterpret_cast<float*>(qp + kQPackScaleOffset);
    sc[tid] = 0.f;
  }
}

struct HistParams {
  const uint8_t* pages;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const float* qrot;
  const float* qsum;
  float* po;
  float* plse;
  int32_t max_pages;
  int32_t hkv;
  int32_t hq;
  const int32_t* sched;
  float lev_lo, lev_hi;   // Lloyd-Max codebook: levels -hi, -lo, lo, hi
  unsigned long long* clk;   // timing hook or nullptr: workgroup (0, 0)'s clock counters
};

// Level of a 2-bit code: the code itself (uniform codebook) or the
// Lloyd-Max level.
template <bool LM>
__device__ __forceinline__ float code_level(uint32_t c, float lo, float hi) {
  if constexpr (LM) {
    const float mag = (c == 0u || c == 3u) ? hi : lo;
    return c >= 2u ? mag : -mag;
  } else {
    return static_cast<float>(c);
  }
}

// Vector-ALU history kernel.  Workgroup = (scheduled split, KV head), four
// waves; wave w takes pages p0+w, p0+w+4, ... of the split with its own
// online-softmax state, and the four states are merged at the end.  LM
// selects the Lloyd-Max codebook (dequantized value zero + scale * level).
template <int GQ, int G, bool LM>
__global__ void __launch_bounds__(256) hist_valu_kernel(HistParams a) {
  constexpr int NG = kDim / G;
  const int split = blockIdx.x, kvh = blockIdx.y;
  if (split >= a.sched[0]) return;   // unused slot (uniform)
  const bool clk = a.clk != nullptr && split == 0 && kvh == 0;   // timing hook (uniform)
  unsigned long long clk0 = 0, wall0 = 0;
  if (clk) {
    clk0 = clock64();
    wall0 = wall_clock64();
  }
  const int b = a.sched[1 + 3 * split];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ float q_s[GQ][kDim];
  __shared__ float qsum_s[GQ][4];
  __shared__ float w_s[4][GQ][NG][kPage];
  __shared__ float st_m[4][GQ], st_l[4][GQ];
  __shared__ float st_acc[4][GQ][kDim];

  const int L = a.seq_lens[b];
  const int n_hist = max(0, L - kBf16Tokens);
  const int p0 = a.sched[2 + 3 * split];
  const int p1 = a.sched[3 + 3 * split];
  const size_t head0 = static_cast<size_t>(b) * a.hq + static_cast<size_t>(kvh) * GQ;
  for (int i = tid; i < GQ * kDim; i += 256) q_s[i / kDim][i % kDim] = a.qrot[head0 * kDim + i];
  if (tid < GQ * 4) qsum_s[tid >> 2][tid & 3] = a.qsum[head0 * 4 + tid];
  __syncthreads();

  float m[GQ], l[GQ], acc0[GQ], acc1[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
    acc0[h] = 0.f;
    acc1[h] = 0.f;
  }
  const int c0 = lane, c1 = lane + 64;
  for (int p = p0 + wave; p < p1; p += 4) {
    const int phys = a.page_table[static_cast<size_t>(b) * a.max_pages + p];
    const uint8_t* blk = a.pages + (static_cast<size_t>(phys) * a.hkv + kvh) * block_bytes(G);
    const uint32_t* words = reinterpret_cast<const uint32_t*>(blk);
    const uint16_t* szk = reinterpret_cast<const uint16_t*>(blk + kCodesBytes);
    const uint16_t* szv = szk + kPage * NG * 2;
    const int t = lane;
    const bool valid = p * kPage + t < n_hist;
    const int qo = qk_order(t);

    // scores: lane = token slot t
    float dot[GQ][NG];
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) dot[h][gi] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t w = words[d * 64 + qo] ^ kTopFieldFlip;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float code = code_level<LM>((w >> (2 * i)) & 3u, a.lev_lo, a.lev_hi);
        const int ch = 16 * d + i;
#pragma unroll
        for (int h = 0; h < GQ; ++h) dot[h][ch / G] = __builtin_fmaf(q_s[h][ch], code, dot[h][ch / G]);
      }
    }
    float sc[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float s = 0.f;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const float ks = bf16_to_f32(szk[(qo * NG + gi) * 2]);
        const float kz = bf16_to_f32(szk[(qo * NG + gi) * 2 + 1]);
        s += ks * dot[h][gi] + kz * qsum_s[h][gi];
      }
      sc[h] = valid ? s : -INFINITY;
    }
    // online softmax over the page
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const float pm = wave_max(sc[h]);
      const float mn = fmaxf(m[h], pm);
      const float alpha = exp2f(m[h] - mn);
      const float pr = valid ? exp2f(sc[h] - mn) : 0.f;
      l[h] = l[h] * alpha + wave_sum(pr);
      m[h] = mn;
      acc0[h] *= alpha;
      acc1[h] *= alpha;
      sc[h] = pr;
    }
    // value weights: p * scale per (head, group, token); zero-point sums
    float u[GQ][NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float vs = valid ? bf16_to_f32(szv[(qo * NG + gi) * 2]) : 0.f;
      const float vz = valid ? bf16_to_f32(szv[(qo * NG + gi) * 2 + 1]) : 0.f;
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        w_s[wave][h][gi][t] = sc[h] * vs;
        u[h][gi] = wave_sum(sc[h] * vz);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // p . v: lane owns channels c0 and c1
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c = half ? c1 : c0;
      const int gi = c / G;
      float accv[GQ];
#pragma unroll
      for (int h = 0; h < GQ; ++h) accv[h] = 0.f;
#pragma unroll
      for (int wq = 0; wq < 4; ++wq) {
        const uint32_t w = words[512 + v_word_index(c, wq)] ^ kTopFieldFlip;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float code = code_level<LM>((w >> (2 * i)) & 3u, a.lev_lo, a.lev_hi);
#pragma unroll
          for (int h = 0; h < GQ; ++h)
            accv[h] = __builtin_fmaf(w_s[wave][h][gi][16 * wq + i], code, accv[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        if (half) acc1[h] += accv[h] + u[h][gi];
        else acc0[h] += accv[h] + u[h][gi];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // merge the four wave states
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    if (lane == 0) {
      st_m[wave][h] = m[h];
      st_l[wave][h] = l[h];
    }
    st_acc[wave][h][c0] = acc0[h];
    st_acc[wave][h][c1] = acc1[h];
  }
  __syncthreads();
  for (int job = tid; job < GQ * kDim; job += 256) {
    const int h = job / kDim, c = job % kDim;
    float mx = -INFINITY;
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, st_m[w][h]);
    float lt = 0.f, at = 0.f;
    if (mx != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        if (st_m[w][h] == -INFINITY) continue;
        const float f = exp2f(st_m[w][h] - mx);
        lt += st_l[w][h] * f;
        at += st_acc[w][h][c] * f;
      }
    }
    const size_t pidx = static_cast<size_t>(split) * a.hq + kvh * GQ + h;
    a.po[pidx * kDim + c] = lt > 0.f ? at / lt : 0.f;
    if (c == 0) a.plse[pidx] = lt > 0.f ? (mx + log2f(lt)) * kLn2 : -INFINITY;
  }
  if (clk && tid == 0) {
    const unsigned long long clk1 = clock64(), wall1 = wall_clock64();
    a.clk[0] = clk0;
    a.clk[1] = wall0;
    a.clk[2] = clk1;
    a.clk[3] = wall1;
  }
}

// Sink + recent as a standalone launch (the matrix-core path runs the same
// chunks inside the history launch).
template <int GQ>
__global__ void __launch_bounds__(64) bf16_kernel(Bf16Params a) {
  __shared__ Bf16Smem<GQ> sm;
  bf16_chunk<GQ>(a, GQ, 0, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

// LSE merge, two launch shapes.  The partial log-sum-exps are natural logs;
// every weight e^(l - max) (argument <= 0) is taken as 2^((l - max) log2 e)
// on the hardware exponential.  merge_head_kernel: workgroup = (query
// head, request), for batches too small to fill the chip by KV head;
// merge_group_kernel: workgroup = (KV head, request), sharing R_V across the
// group's heads.
//
// merge_head_kernel (kMergeHeadThreads = 1024 threads): the request's
// history splits (from the schedule) are merged in the rotated value domain,
// rotated back by R_V^T, and merged with the five bf16 partials.  Thread t
// weighs split t; the weighted sum over splits runs on eight threads per
// channel (channel t % 128, every eighth split: up to 32 loads per thread
// for a long request's 251 splits); each thread holds an eighth of a row of
// R_V, loaded before anything else.
struct MergeParams {
  const float* ho;        // [slots][Hq][128]
  const float* hlse;      // [slots][Hq]
  const float* bo;        // [B][Hq][5][128]
  const float* blse;      // [B][Hq][5]
  const int32_t* req;     // [B][2] {first split, count}
  const float* r_v;
  float* out;
  float* lse_out;
  int32_t hq;
  int32_t gq;
};

#ifndef OSCAR_MERGE_HEAD_THREADS
#define OSCAR_MERGE_HEAD_THREADS 1024
#endif
constexpr int kMergeHeadThreads = OSCAR_MERGE_HEAD_THREADS;
static_assert(kMaxSplits < kMergeHeadThreads, "one thread weighs each split");

__global__ void __launch_bounds__(kMergeHeadThreads) merge_head_kernel(MergeParams a) {
  constexpr int kWaves = kMergeHeadThreads / 64;
  constexpr int kPar = kMergeHeadThreads / kDim;   // threads per channel
  constexpr int kPer = (kMaxSplits + kPar - 1) / kPar;   // history partials per thread
  static_assert(kPer * kPar >= kMaxSplits, "every split has a thread");
  const int head = blockIdx.x, b = blockIdx.y, kvh = head / a.gq;
  const int tid = threadIdx.x;
  __shared__ float red[kWaves];
  __shared__ float w[kMaxSplits + 1];
  __shared__ float ypart[kPar][kDim];
  __shared__ float y[kDim];
  auto bmax = [&](float v) {
    v = wave_max(v);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r = fmaxf(r, red[i]);
    return r;
  };
  auto bsum = [&](float v) {
    v = wave_sum(v);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r += red[i];
    return r;
  };
  const int first = a.req[2 * b], count = a.req[2 * b + 1];
  const size_t bh = static_cast<size_t>(b) * a.hq + head;
  // the log-sum-exps first: the weights need only these
  // (loads unconditional with clamped indices, values selected afterwards:
  // a conditional load becomes a branch whose wait serialises the loads)
  const int last_sp = max(count - 1, 0);
  const size_t slot0 = count > 0 ? static_cast<size_t>(first) : 0;
  const float l_raw = a.hlse[(slot0 + min(tid, last_sp)) * a.hq + head];
  const float l = tid < count ? l_raw : -INFINITY;
  float lb[kBf16Parts];
#pragma unroll
  for (int c = 0; c < kBf16Parts; ++c) lb[c] = a.blse[bh * kBf16Parts + c];
  // thread (i, kh): row i of R_V, columns kCols kh .. kCols (kh + 1) - 1
  constexpr int kParts = kMergeHeadThreads / kDim, kCols = kDim / kParts;
  static_assert(kParts == 4 || kParts == 8, "four or eight threads per R_V row");
  const int i = tid / kParts, kh = tid % kParts;
  float4 rr[kCols / 4];
  {
    const float4* rrow =
        reinterpret_cast<const float4*>(a.r_v + (static_cast<size_t>(kvh) * kDim + i) * kDim + kCols * kh);
#pragma unroll
    for (int c = 0; c < kCols / 4; ++c) rr[c] = rrow[c];
  }
  // every history partial this thread sums (channel k, the splits congruent
  // to par modulo kPar) and its bf16 partials are requested now, before the
  // weights are known, so the kernel waits on memory once
  const int k = tid & (kDim - 1), par = tid / kDim;
  const float* hp = a.ho + (slot0 * a.hq + head) * kDim + k;
  const size_t stride = static_cast<size_t>(a.hq) * kDim;
  float v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int sp = par + kPar * u;
    const float x = hp[static_cast<size_t>(min(sp, last_sp)) * stride];
    v[u] = sp < count ? x : 0.f;
  }
  float vb[kBf16Parts];
#pragma unroll
  for (int c = 0; c < kBf16Parts; ++c) {
    const float x = a.bo[(bh * kBf16Parts + c) * kDim + i];
    vb[c] = kh == 0 ? x : 0.f;
  }
  // history split weights e^{lse - M} / sum (count <= kMaxSplits < threads)
  const float mh = bmax(l);
  const float e = mh == -INFINITY || tid >= count ? 0.f : __builtin_amdgcn_exp2f((l - mh) * kLog2e);
  const float dh = bsum(e);
  if (tid < count) w[tid] = dh > 0.f ? e / dh : 0.f;
  const float lse_h = dh > 0.f ? mh + logf(dh) : -INFINITY;
  // bf16 partial weights (every thread computes the five)
  float mb = -INFINITY;
#pragma unroll
  for (int c = 0; c < kBf16Parts; ++c) mb = fmaxf(mb, lb[c]);
  float db = 0.f;
#pragma unroll
  for (int c = 0; c < kBf16Parts; ++c)
    db += lb[c] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lb[c] - mb) * kLog2e);
  const float lse_b = mb + logf(db);   // the sink chunk always holds a token
  __syncthreads();
  // weighted sum over the splits, in ascending split order
  {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int sp = par + kPar * u;
      if (sp < count) acc = __builtin_fmaf(w[sp], v[u], acc);
    }
    ypart[par][k] = acc;
  }
  __syncthreads();
  if (tid < kDim) {
    float t = 0.f;
#pragma unroll
    for (int p = 0; p < kPar; ++p) t += ypart[p][tid];
    y[tid] = t;
  }
  __syncthreads();
  // back to the model domain: x_i = sum_k y_k R_V[i][k]
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < kCols / 4; ++c) {
    const int kc = kCols * kh + 4 * c;
    acc = __builtin_fmaf(y[kc + 0], rr[c].x, acc);
    acc = __builtin_fmaf(y[kc + 1], rr[c].y, acc);
    acc = __builtin_fmaf(y[kc + 2], rr[c].z, acc);
    acc = __builtin_fmaf(y[kc + 3], rr[c].w, acc);
  }
#pragma unroll
  for (int o = 1; o < kParts; o <<= 1) acc += __shfl_xor(acc, o, 64);
  const float xh = acc;
  if (kh == 0) {
    float ob = 0.f;
#pragma unroll
    for (int c = 0; c < kBf16Parts; ++c) {
      const float wc = lb[c] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lb[c] - mb) * kLog2e) / db;
      ob = __builtin_fmaf(wc, vb[c], ob);
    }
    const float mx = fmaxf(lse_h, lse_b);
    const float eh = lse_h == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lse_h - mx) * kLog2e);
    const float eb = __builtin_amdgcn_exp2f((lse_b - mx) * kLog2e);
    const float den = eh + eb;
    a.out[bh * kDim + i] = (eh * xh + eb * ob) / den;
    if (a.lse_out != nullptr && i == 0) a.lse_out[bh] = mx + logf(den);
  }
}

// merge_group_kernel (kMergeGroupThreads = 512 threads, one (head,
// channel) item per thread for four-head blocks): the request's history splits are
// merged per head in the rotated value domain, rotated back by R_V^T, and
// merged with the five bf16 partials.  A workgroup takes GQ heads of one
// (request, KV head): heads GQ * blockIdx.z .. of the group (eight-head
// groups run as two four-head workgroups).  Each thread owns (head,
// channel) items and, for the un-rotation, half a row of R_V.
//
// Loads are issued in the order they are needed: the log-sum-exps and the
// partials of the first 16 splits and of the bf16 chunks, then R_V, so the
// weights do not wait for the rotation rows.  When a request has at most 16
// splits (the usual case at large batch) every thread computes its heads'
// weights itself from the log-sum-exps it loaded (the same few addresses
// across a wave): no reductions across lanes and one workgroup barrier.
// Longer requests take the cooperative path: weights per head by one wave
// through LDS, partials past the 16th read 16 at a time.
template <int GQ, int NT>
__global__ void __launch_bounds__(NT) merge_group_kernel(MergeParams a) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int kMaxHist = kMaxSplits + 1;
  __shared__ float wh[GQ][kMaxHist];   // history split weights (cooperative path)
  __shared__ float wb[GQ][kBf16Parts]; // bf16 partial weights (cooperative path)
  __shared__ float lse_s[GQ][2];       // history LSE, bf16 LSE
  __shared__ float orot[GQ][kDim];     // merged history output, rotated domain
  __shared__ float obf[GQ][kDim];      // merged bf16 output
  const int first = a.req[2 * b], count = a.req[2 * b + 1];
  const int h0 = kvh * a.gq + GQ * static_cast<int>(blockIdx.z);   // first head of this workgroup's block
  const size_t bhead0 = static_cast<size_t>(b) * a.hq + h0;
  constexpr int kItems = (GQ * kDim + NT - 1) / NT;   // (head, channel) items per thread
  constexpr int kEarly = 16;
  // (kept for up to two items per thread: four or more per thread would hold
  // twice the registers and spill)
  const bool local = kItems <= 2 && count <= kEarly;   // uniform
  const size_t hstride = static_cast<size_t>(a.hq) * kDim;
  constexpr int kLocalItems = kItems <= 2 ? kItems : 1;
  float vh[kItems][kEarly], vb[kItems][kBf16Parts], lh[kLocalItems][kEarly], lb[kLocalItems][kBf16Parts];
  // Every load is issued unconditionally, its index clamped to one that
  // exists, and its value selected afterwards: a load under a condition
  // compiles to a branch around it, and the wait at each branch serialised
  // the loads (a request's first split slot is `first` only when it has
  // history)
  const int last_u = max(count - 1, 0);
  const size_t slot0 = count > 0 ? static_cast<size_t>(first) : 0;
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int x = tid + NT * it;
    const bool live = x < GQ * kDim;
    const int xc = live ? x : 0;
    const int h = xc / kDim, k = xc % kDim;
    const float* hb = a.ho + (slot0 * a.hq + h0 + h) * kDim + k;
    // (masks applied arithmetically: the loaded values are finite, and a
    // select on them let the compiler move each load under a branch)
#pragma unroll
    for (int u = 0; u < kEarly; ++u) {
      const float v = hb[static_cast<size_t>(min(u, last_u)) * hstride];
      vh[it][u] = v * (live && u < count ? 1.f : 0.f);
    }
    const float* bb = a.bo + ((bhead0 + h) * kBf16Parts) * kDim + k;
#pragma unroll
    for (int c = 0; c < kBf16Parts; ++c) vb[it][c] = bb[c * kDim] * (live ? 1.f : 0.f);
    if constexpr (kItems <= 2) {   // loaded whether or not the request takes the local path
      // a wave's items share one head (128 channels = two waves), so its
      // log-sum-exps are wave-uniform: scalar loads, outside the vector
      // load count
      const int hu = __builtin_amdgcn_readfirstlane(h);
#pragma unroll
      for (int u = 0; u < kEarly; ++u) {
        const float l = a.hlse[(slot0 + min(u, last_u)) * a.hq + h0 + hu];
        lh[it][u] = l + (live && u < count ? 0.f : -INFINITY);
      }
#pragma unroll
      for (int c = 0; c < kBf16Parts; ++c)
        lb[it][c] = a.blse[(bhead0 + hu) * kBf16Parts + c] + (live ? 0.f : -INFINITY);
    }
  }
  if (!local) {
    for (int x = tid; x < GQ * count; x += NT) {
      const int h = x / count, sp = x % count;
      wh[h][sp] = a.hlse[static_cast<size_t>(first + sp) * a.hq + h0 + h];
    }
    for (int x = tid; x < GQ * kBf16Parts; x += NT)
      wb[x / kBf16Parts][x % kBf16Parts] = a.blse[(bhead0 + x / kBf16Parts) * kBf16Parts + x % kBf16Parts];
  }
  // thread (i, kh): row i of R_V, columns kCols kh .. kCols (kh + 1) - 1
  constexpr int kParts = NT / kDim, kCols = kDim / kParts;
  static_assert(kParts == 2 || kParts == 4, "two or four threads per R_V row");
  const int i = tid / kParts, kh = tid % kParts;
  float4 rr[kCols / 4];
  const float4* rrow =
      reinterpret_cast<const float4*>(a.r_v + (static_cast<size_t>(kvh) * kDim + i) * kDim + kCols * kh);
#pragma unroll
  for (int c = 0; c < kCols / 4; ++c) rr[c] = rrow[c];
  if (local) {
    // each thread weighs its own items' partials
#pragma unroll
    for (int it = 0; it < kLocalItems; ++it) {
      const int x = tid + NT * it;
      if (x >= GQ * kDim) break;
      const int h = x / kDim, k = x % kDim;
      float mh = -INFINITY;
#pragma unroll
      for (int u = 0; u < kEarly; ++u) mh = fmaxf(mh, lh[it][u]);
      float dh = 0.f, oh = 0.f;
#pragma unroll
      // (e^x as 2^(x log2 e) on the hardware exponential: arguments <= 0,
      // and -inf gives 0)
      for (int u = 0; u < kEarly; ++u) {
        const float e = u < count && mh != -INFINITY ? __builtin_amdgcn_exp2f((lh[it][u] - mh) * kLog2e) : 0.f;
        dh += e;
        oh = __builtin_fmaf(e, vh[it][u], oh);
      }
      float mb = -INFINITY;
#pragma unroll
      for (int c = 0; c < kBf16Parts; ++c) mb = fmaxf(mb, lb[it][c]);
      float db = 0.f, ob = 0.f;
#pragma unroll
      for (int c = 0; c < kBf16Parts; ++c) {
        const float e = lb[it][c] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lb[it][c] - mb) * kLog2e);
        db += e;
        ob = __builtin_fmaf(e, vb[it][c], ob);
      }
      orot[h][k] = dh > 0.f ? oh / dh : 0.f;
      obf[h][k] = db > 0.f ? ob / db : 0.f;
      if (k == 0) {
        lse_s[h][0] = dh > 0.f ? mh + logf(dh) : -INFINITY;
        lse_s[h][1] = db > 0.f ? mb + logf(db) : -INFINITY;
      }
    }
  } else {
    __syncthreads();
    // per head and side: normalised weights of the partials
    for (int h = wave; h < GQ; h += NT / 64) {
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        float* w = side ? wb[h] : wh[h];
        const int n = side ? kBf16Parts : count;
        float mx = -INFINITY;
        for (int sp = lane; sp < n; sp += 64) mx = fmaxf(mx, w[sp]);
        mx = wave_max(mx);
        float den = 0.f;
        for (int sp = lane; sp < n; sp += 64)
          den += mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((w[sp] - mx) * kLog2e);
        den = wave_sum(den);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int sp = lane; sp < n; sp += 64)
          w[sp] = den > 0.f ? __builtin_amdgcn_exp2f((w[sp] - mx) * kLog2e) / den : 0.f;
        if (lane == 0) lse_s[h][side] = den > 0.f ? mx + logf(den) : -INFINITY;
      }
    }
    __syncthreads();
    // weighted sums of the partials: the first 16 splits from registers, the
    // rest 16 loads at a time
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int x = tid + NT * it;
      if (x >= GQ * kDim) break;
      const int h = x / kDim, k = x % kDim;
      float oh = 0.f;
#pragma unroll
      for (int u = 0; u < kEarly; ++u)
        if (u < count) oh = __builtin_fmaf(wh[h][u], vh[it][u], oh);
      const float* hb = a.ho + (static_cast<size_t>(first) * a.hq + h0 + h) * kDim + k;
      for (int s0 = kEarly; s0 < count; s0 += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = s0 + u < count ? hb[static_cast<size_t>(s0 + u) * hstride] : 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (s0 + u < count) oh = __builtin_fmaf(wh[h][s0 + u], v[u], oh);
      }
      float ob = 0.f;
#pragma unroll
      for (int c = 0; c < kBf16Parts; ++c) ob = __builtin_fmaf(wb[h][c], vb[it][c], ob);
      orot[h][k] = oh;
      obf[h][k] = ob;
    }
  }
  __syncthreads();
  // history output back to the model domain: x_i = sum_k y_k R_V[i][k]
  float oh[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < kCols / 4; ++c) {
      const int k = kCols * kh + 4 * c;
      acc = __builtin_fmaf(orot[h][k + 0], rr[c].x, acc);
      acc = __builtin_fmaf(orot[h][k + 1], rr[c].y, acc);
      acc = __builtin_fmaf(orot[h][k + 2], rr[c].z, acc);
      acc = __builtin_fmaf(orot[h][k + 3], rr[c].w, acc);
    }
    acc += __shfl_xor(acc, 1, 64);
    if constexpr (kParts == 4) acc += __shfl_xor(acc, 2, 64);
    oh[h] = acc;
  }
  if (kh == 0) {
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      const float lh = lse_s[h][0], lbb = lse_s[h][1];
      const float mx = fmaxf(lh, lbb);
      const float whh = lh == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lh - mx) * kLog2e);
      const float wbb = lbb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lbb - mx) * kLog2e);
      const float den = whh + wbb;
      a.out[(bhead0 + h) * kDim + i] = den > 0.f ? (whh * oh[h] + wbb * obf[h][i]) / den : 0.f;
      if (a.lse_out != nullptr && i == 0) a.lse_out[bhead0 + h] = den > 0.f ? mx + logf(den) : -INFINITY;
    }
  }
}

template <template <int> class F, typename... Args>
hipError_t dispatch_gq(int gq, Args... args) {
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

// Weight ratio of the Lloyd-Max high-bit plane to the code plane in the
// matrix-core kernel ((3 lo - hi) / 2 over hi - lo); 0 for the uniform
// codebook (no second operand).
inline float lm_ratio(const oscar_dims& d) {
  if (d.codebook != OSCAR_CODEBOOK_LLOYD_MAX) return 0.f;
  const Codebook* c = codebook_of(d.codebook);
  return (3.f * c->lev[2] - c->lev[3]) * 0.5f / (c->lev[3] - c->lev[2]);
}

template <int GQ>
struct QrotRun {
  static hipError_t run(const DecodeArgs& a, hipStream_t s) {
    const oscar_dims& d = *a.dims;
    const int batch = a.cache->batch;
    // the demotion rows: one 256-thread workgroup each for the key and the
    // value while the launch is small (batch 1 x 8 KV heads: 33.4/33.7 ->
    // 33.0/33.1 us per step), the key and value halves of one workgroup
    // otherwise (at 32 x 8 the doubled rows cost the step about 1 us)
    const bool wide = batch * d.num_kv_heads <= 64;
    const dim3 grid(d.num_kv_heads, 1 + batch + (a.demote != nullptr ? (wide ? 2 : 1) * batch : 0));
    qrot_kernel<GQ><<<grid, 256, 0, s>>>(
        a.q, a.rot->r_k, d.num_q_heads, d.num_kv_heads, d.group_size,
        reinterpret_cast<float*>(a.ws + a.lay.off_qrot), reinterpret_cast<float*>(a.ws + a.lay.off_qsum),
        a.ws + a.lay.off_qpack, a.cache->seq_lens, batch, a.sched_target > 0 ? a.sched_target : a.lay.target,
        reinterpret_cast<int32_t*>(a.ws + a.lay.off_sched), reinterpret_cast<int32_t*>(a.ws + a.lay.off_req),
        lm_ratio(d), a.demote != nullptr ? *a.demote : DemoteStep{});
    return hipGetLastError();
  }
};

template <int GQ>
struct HistValuRun {
  static hipError_t run(const DecodeArgs& a, hipStream_t s) {
    const oscar_dims& d = *a.dims;
    HistParams p;
    p.pages = a.cache->pages;
    p.page_table = a.cache->page_table;
    p.seq_lens = a.cache->seq_lens;
    p.qrot = reinterpret_cast<const float*>(a.ws + a.lay.off_qrot);
    p.qsum = reinterpret_cast<const float*>(a.ws + a.lay.off_qsum);
    p.po = reinterpret_cast<float*>(a.ws + a.lay.off_ho);
    p.plse = reinterpret_cast<float*>(a.ws + a.lay.off_hlse);
    p.max_pages = a.cache->max_pages_per_req;
    p.hkv = d.num_kv_heads;
    p.hq = d.num_q_heads;
    p.sched = reinterpret_cast<const int32_t*>(a.ws + a.lay.off_sched);
    const Codebook* cb = codebook_of(d.codebook);
    p.lev_lo = cb->lev[2];
    p.lev_hi = cb->lev[3];
    p.clk = a.clock_trace;
    const dim3 grid(a.lay.slots, d.num_kv_heads);
    const bool timed = a.ev_start != nullptr && a.ev_stop != nullptr;
    if (d.codebook == OSCAR_CODEBOOK_LLOYD_MAX) {
      switch (d.group_size) {
        case 32: launch(hist_valu_kernel<GQ, 32, true>, grid, timed, a, p, s); break;
        case 64: launch(hist_valu_kernel<GQ, 64, true>, grid, timed, a, p, s); break;
        default: launch(hist_valu_kernel<GQ, 128, true>, grid, timed, a, p, s); break;
      }
    } else {
      switch (d.group_size) {
        case 32: launch(hist_valu_kernel<GQ, 32, false>, grid, timed, a, p, s); break;
        case 64: launch(hist_valu_kernel<GQ, 64, false>, grid, timed, a, p, s); break;
        default: launch(hist_valu_kernel<GQ, 128, false>, grid, timed, a, p, s); break;
      }
    }
    return hipGetLastError();
  }
  template <typename K>
  static void launch(K kernel, dim3 grid, bool timed, const DecodeArgs& a, const HistParams& p, hipStream_t s) {
    if (timed)
      hipExtLaunchKernelGGL(kernel, grid, dim3(256), 0, s, a.ev_start, a.ev_stop, 0, p);
    else
      kernel<<<grid, 256, 0, s>>>(p);
  }
};

template <int GQ>
struct Bf16Run {
  static hipError_t run(const DecodeArgs& a, hipStream_t s) {
    const oscar_dims& d = *a.dims;
    const Bf16Params p = make_bf16_params(a);
    const dim3 grid(kBf16Parts, d.num_kv_heads, a.cache->batch);
    bf16_kernel<GQ><<<grid, 64, 0, s>>>(p);
    return hipGetLastError();
  }
};

#ifndef OSCAR_MERGE_GROUP_THREADS
#define OSCAR_MERGE_GROUP_THREADS 512
#endif
constexpr int kMergeGroupThreads = OSCAR_MERGE_GROUP_THREADS;

template <int GQ>
struct MergeGroupRun {
  static hipError_t run(const MergeParams& p, int hkv, int32_t batch, hipStream_t s) {
    merge_group_kernel<GQ, kMergeGroupThreads><<<dim3(hkv, batch), kMergeGroupThreads, 0, s>>>(p);
    return hipGetLastError();
  }
};

// Below this many (request, KV head) workgroups the merge runs one
// workgroup per query head.
constexpr int kMergeGroupMinWgs = 128;

}  // namespace

hipError_t launch_qrot(const DecodeArgs& a, hipStream_t s) {
  return dispatch_gq<QrotRun>(a.dims->num_q_heads / a.dims->num_kv_heads, a, s);
}

hipError_t launch_hist_valu(const DecodeArgs& a, hipStream_t s) {
  return dispatch_gq<HistValuRun>(a.dims->num_q_heads / a.dims->num_kv_heads, a, s);
}

hipError_t launch_bf16(const DecodeArgs& a, hipStream_t s) {
  return dispatch_gq<Bf16Run>(a.dims->num_q_heads / a.dims->num_kv_heads, a, s);
}

hipError_t launch_merge(const oscar_dims& d, const oscar_rotation& rot, int32_t batch,
                        const uint8_t* ws, const WsLayout& lay, float* out, float* lse_out,
                        hipStream_t s) {
  MergeParams p;
  p.ho = reinterpret_cast<const float*>(ws + lay.off_ho);
  p.hlse = reinterpret_cast<const float*>(ws + lay.off_hlse);
  p.bo = reinterpret_cast<const float*>(ws + lay.off_bo);
  p.blse = reinterpret_cast<const float*>(ws + lay.off_blse);
  p.req = reinterpret_cast<const int32_t*>(ws + lay.off_req);
  p.r_v = rot.r_v;
  p.out = out;
  p.lse_out = lse_out;
  p.hq = d.num_q_heads;
  p.gq = d.num_q_heads / d.num_kv_heads;
  if (static_cast<int64_t>(batch) * d.num_kv_heads < kMergeGroupMinWgs) {
    merge_head_kernel<<<dim3(d.num_q_heads, batch), kMergeHeadThreads, 0, s>>>(p);
    return hipGetLastError();
  }
  if (p.gq % 4 == 0 && p.gq > 4) {   // four heads per workgroup: more, shorter workgroups
    merge_group_kernel<4, kMergeGroupThreads><<<dim3(d.num_kv_heads, batch, p.gq / 4), kMergeGroupThreads, 0, s>>>(
        p);
    return hipGetLastError();
  }
  return dispatch_gq<MergeGroupRun>(p.gq, p, d.num_kv_heads, batch, s);
}

}  // namespace oscar
