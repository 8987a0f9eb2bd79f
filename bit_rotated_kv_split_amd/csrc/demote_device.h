// Demotion device code shared by the demotion and decode-prologue kernels:
// rotate, clip, quantize and pack tokens into history page blocks (page
// "超越TurboQuant：Together AI把2-bit KV Cache推向真实服务", section
// "OSCAR的另一个关键点是"; the quantizer of the first page, section
// "为什么 INT2 KV 缓存量化很难？"; the Lloyd-Max codebook that the second
// page's comparison with TurboQuant mentions).
#pragma once

#include "oscar_device.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr int kMaxChunk = 16;

// Shared memory of one 128-thread demotion unit (sized for the smallest
// group, G = 32, so one type serves every G).
template <int NT>
struct QuantSmem {
  static constexpr int kMaxNG = kDim / 32;
  float x[NT][kDim];
  float y[NT][kDim];
  float scale[NT][kMaxNG];
  float zero[NT][kMaxNG];
  float xw[2][NT][2];          // per-wave (min, max) when a group spans both waves
  double xd[2][2][NT];         // per-wave float64 (sum, sum of squares), same case
  uint8_t code[NT][kDim];
  double rp[8][kDim];          // demotion of one token: float64 partial rotations per row group
};

// Sum over the G lanes of this thread's group, in float64: a butterfly
// inside the wave, then (G = 128) the two waves' halves through LDS.  Every
// thread of the 128-thread unit calls it.
template <int G, int NT>
__device__ __forceinline__ void group_sum_f64(double (&v)[NT], double (&xd)[2][NT], int lane, int wave) {
  constexpr int WG = G < 64 ? G : 64;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int off = 1; off < WG; off <<= 1) v[t] += __shfl_xor(v[t], off, 64);
  if constexpr (G == 128) {
    if (lane == 0)
#pragma unroll
      for (int t = 0; t < NT; ++t) xd[wave][t] = v[t];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = xd[0][t] + xd[1][t];
  }
}

// The quantizers:
//   OSCAR_CODEBOOK_UNIFORM: zero = bf16(min), scale = bf16((max - min) / 3),
//     code = clamp(rint((y - zero) / scale), 0, 3).
//   OSCAR_CODEBOOK_LLOYD_MAX: zero = bf16(float(mean)), scale =
//     bf16(float(population standard deviation)), mean and deviation in
//     float64; code = number of thresholds (-thr, 0, thr) below
//     (y - zero) / scale.
// A group whose scale is 0 gets code 0.
template <int G, int NT>
__device__ void quantize_rotated(QuantSmem<NT>& sm, int nt, float (&y)[NT], int k, int codebook, float thr);

// Rotate, clip and quantize nt tokens held in sm.x (see quantize_rotated).
template <int G, int NT>
__device__ void quantize_tokens(QuantSmem<NT>& sm, int nt, const float* __restrict__ r,
                                const float* __restrict__ clipv, int k, int codebook, float thr) {
  double acc[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = 0.0;
  for (int i = 0; i < kDim; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const double rik = static_cast<double>(r[(i + u) * kDim + k]);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][u] = fma(static_cast<double>(sm.x[t][i + u]), rik, acc[t][u]);
    }
  }
  const float c = clipv[k];
  float y[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const double sum = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
    y[t] = fminf(fmaxf(static_cast<float>(sum), -c), c);
  }
  quantize_rotated<G, NT>(sm, nt, y, k, codebook, thr);
}

// Quantize nt (<= NT) rotated, clipped tokens, channel k of token t in y[t].
// Called by the 128 threads of one unit (k = 0..127, two whole waves);
// every thread of the workgroup passes the same barriers (the codebook is
// uniform across it).  Leaves codes, scale and zero in sm.
template <int G, int NT>
__device__ void quantize_rotated(QuantSmem<NT>& sm, int nt, float (&y)[NT], int k, int codebook, float thr) {
  constexpr int WG = G < 64 ? G : 64;   // group lanes inside one wave
  const int lane = k & 63, wave = k >> 6;
  auto& xw = sm.xw;
#pragma unroll
  for (int t = 0; t < NT; ++t) sm.y[t][k] = y[t];
  const int gi = k / G;
  if (codebook == OSCAR_CODEBOOK_LLOYD_MAX) {
    double mean[NT], sq[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) mean[t] = static_cast<double>(y[t]);
    group_sum_f64<G, NT>(mean, sm.xd[0], lane, wave);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      mean[t] /= G;
      const double d = static_cast<double>(y[t]) - mean[t];
      sq[t] = d * d;
    }
    group_sum_f64<G, NT>(sq, sm.xd[1], lane, wave);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float s = bf16_round(static_cast<float>(sqrt(sq[t] / G)));
      const float z = bf16_round(static_cast<float>(mean[t]));
      if (k % G == 0 && t < nt) {
        sm.scale[t][gi] = s;
        sm.zero[t][gi] = z;
      }
      int code = 0;
      if (s != 0.f) {
        const float u = (y[t] - z) / s;
        code = (u > -thr) + (u > 0.f) + (u > thr);
      }
      if (t < nt) sm.code[t][k] = static_cast<uint8_t>(code);
    }
    __syncthreads();
    return;
  }
  // group min / max across the G lanes of a group
  float mn[NT], mx[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    mn[t] = y[t];
    mx[t] = y[t];
#pragma unroll
    for (int off = 1; off < WG; off <<= 1) {
      mn[t] = fminf(mn[t], __shfl_xor(mn[t], off, 64));
      mx[t] = fmaxf(mx[t], __shfl_xor(mx[t], off, 64));
    }
  }
  if constexpr (G == 128) {
    if (lane == 0)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        xw[wave][t][0] = mn[t];
        xw[wave][t][1] = mx[t];
      }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      mn[t] = fminf(xw[0][t][0], xw[1][t][0]);
      mx[t] = fmaxf(xw[0][t][1], xw[1][t][1]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float range = mx[t] - mn[t];
    const float s = bf16_round(range / 3.0f);
    const float z = bf16_round(mn[t]);
    if (k % G == 0 && t < nt) {
      sm.scale[t][gi] = s;
      sm.zero[t][gi] = z;
    }
    int code = 0;
    if (s != 0.f) {
      const float diff = y[t] - z;
      const float q = rintf(diff / s);
      code = static_cast<int>(fminf(fmaxf(q, 0.f), 3.f));
    }
    if (t < nt) sm.code[t][k] = static_cast<uint8_t>(code);
  }
  __syncthreads();
}

// Store nt quantized tokens occupying slots slot0 .. slot0+nt-1 of one page
// block (all inside one 16-slot value word).  is_v selects the value half.
template <int G, int NT>
__device__ void store_tokens(const QuantSmem<NT>& sm, int nt, uint8_t* __restrict__ blk,
                             int slot0, bool is_v, int k) {
  constexpr int NG = kDim / G;
  uint32_t* words = reinterpret_cast<uint32_t*>(blk);
  if (!is_v) {
    for (int job = k; job < nt * 8; job += kDim) {
      const int t = job >> 3, d = job & 7;
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) w |= static_cast<uint32_t>(sm.code[t][16 * d + i]) << (2 * i);
      words[d * 64 + qk_order(slot0 + t)] = w ^ kTopFieldFlip;
    }
  } else {
    // channel k: one value word holds slots 16w..16w+15 of this channel
    const int w = slot0 >> 4;
    uint32_t bits = 0, mask = 0;
    for (int t = 0; t < nt; ++t) {
      const int sh = 2 * ((slot0 + t) & 15);
      bits |= code_bits(sm.code[t][k], (slot0 + t) & 15);
      mask |= 3u << sh;
    }
    uint32_t* wp = words + 512 + v_word_index(k, w);
    const uint32_t old = (mask == 0xFFFFFFFFu) ? 0u : *wp;
    *wp = (old & ~mask) | bits;
  }
  uint16_t* sz = reinterpret_cast<uint16_t*>(blk + kCodesBytes + (is_v ? kPage * NG * 4 : 0));
  for (int job = k; job < nt * NG; job += kDim) {
    const int t = job / NG, gi = job % NG;
    uint16_t* e = sz + (qk_order(slot0 + t) * NG + gi) * 2;
    e[0] = f32_to_bf16_rne(sm.scale[t][gi]);
    e[1] = f32_to_bf16_rne(sm.zero[t][gi]);
  }
}

// Demotion of one (request, KV head, K or V) for a decode step, by one
// unit of NT = 128 or 256 threads (thread k): the token at position L-257 leaves the recent
// ring for history index L-321, then the new token (if given) takes its
// sink or recent slot.  Everything the unit reads is requested right after
// the length, so the unit waits on memory about twice (the length, then
// the token, its rotation column, the clip threshold, the page-table entry
// and the new token together); the value word's other fifteen slots are
// kept by an atomic AND/OR pair instead of a read-modify-write.  With
// 256 threads each thread sums half as many rows of R; both halves then
// run the quantizer on the same values (identical LDS writes) and only the
// first half stores.
template <int G, int NT = kDim>
__device__ void demote_unit(const DemoteStep& d, int kvh, int b, bool is_v, int kt, QuantSmem<1>& sm) {
  static_assert(NT == kDim || NT == 2 * kDim, "one or two threads per channel");
  constexpr int NG = kDim / G;
  constexpr int kRG = NT / 32, kRows = kDim / kRG;   // row groups, rows per group
  const int k = kt & (kDim - 1);                     // channel
  const bool writer = kt < kDim;                     // uniform per wave
  const DemoteArgs& a = is_v ? d.vv : d.kk;
  const int hkv = a.hkv;
  const int L = d.seq_lens[b];
  uint16_t* recent = (is_v ? d.recent_v : d.recent_k) + (static_cast<size_t>(b) * hkv + kvh) * kRecent * kDim;
  const uint16_t* src = is_v ? d.v_new : d.k_new;
  const bool append = src != nullptr && L >= 1;   // uniform across the workgroup
  const uint16_t val = append && writer ? src[(static_cast<size_t>(b) * hkv + kvh) * kDim + k] : uint16_t{0};
  if (L > kBf16Tokens) {   // uniform across the workgroup
    const int j = L - kBf16Tokens - 1;            // history index of position L-257
    const int ring = (L - 1 - kSink) & (kRecent - 1);
    // x . R: thread kt sums rows kRows rg .. kRows rg + kRows - 1
    // (rg = kt / 32) for channels 4 cq .. 4 cq + 3 (cq = kt % 32), float64
    // products, 16-byte loads of R; the row-group partials of channel k are
    // added in a fixed order and rounded once to float32
    const int cq = kt & 31, rg = kt >> 5;
    const float4* r4 = reinterpret_cast<const float4*>(a.r + static_cast<size_t>(kvh) * kDim * kDim);
    const uint16_t xk = recent[ring * kDim + k];
    float4 rv[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) rv[i] = r4[(kRows * rg + i) * (kDim / 4) + cq];
    const float c = a.clip[kvh * kDim + k];
    const int phys = a.page_table[static_cast<size_t>(b) * a.max_pages + (j >> 6)];
    if (writer) sm.x[0][k] = bf16_to_f32(xk);
    __syncthreads();
    {
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        const double xi = static_cast<double>(sm.x[0][kRows * rg + i]);
        acc[0] = fma(xi, static_cast<double>(rv[i].x), acc[0]);
        acc[1] = fma(xi, static_cast<double>(rv[i].y), acc[1]);
        acc[2] = fma(xi, static_cast<double>(rv[i].z), acc[2]);
        acc[3] = fma(xi, static_cast<double>(rv[i].w), acc[3]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.rp[rg][4 * cq + e] = acc[e];
    }
    __syncthreads();
    double ys = (sm.rp[0][k] + sm.rp[1][k]) + (sm.rp[2][k] + sm.rp[3][k]);
    if constexpr (kRG == 8) ys += (sm.rp[4][k] + sm.rp[5][k]) + (sm.rp[6][k] + sm.rp[7][k]);
    const float yk = static_cast<float>(ys);
    float y[1] = {fminf(fmaxf(yk, -c), c)};
    quantize_rotated<G, 1>(sm, 1, y, k, a.codebook, a.thr);
    uint8_t* blk = a.pages + (static_cast<size_t>(phys) * hkv + kvh) * block_bytes(G);
    const int slot = j & 63;
    if (!writer) return;   // the second half has no stores; nothing below waits
    uint32_t* words = reinterpret_cast<uint32_t*>(blk);
    if (!is_v) {
      if (k < 8) {   // key word d = k: channels 16k .. 16k+15 of this slot
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) w |= static_cast<uint32_t>(sm.code[0][16 * k + i]) << (2 * i);
        words[k * 64 + qk_order(slot)] = w ^ kTopFieldFlip;
      }
    } else {
      // channel k's value word holds slots 16w .. 16w+15: clear this slot's
      // two bits, then set them (same address, same thread: in order)
      uint32_t* wp = words + 512 + v_word_index(k, slot >> 4);
      const int sh = 2 * (slot & 15);
      atomicAnd(wp, ~(3u << sh));
      atomicOr(wp, code_bits(sm.code[0][k], slot & 15));
    }
    if (k < NG) {
      uint16_t* e = reinterpret_cast<uint16_t*>(blk + kCodesBytes + (is_v ? kPage * NG * 4 : 0)) +
                    (qk_order(slot) * NG + k) * 2;
      e[0] = f32_to_bf16_rne(sm.scale[0][k]);
      e[1] = f32_to_bf16_rne(sm.zero[0][k]);
    }
  }
  if (append && writer) {
    const int p = L - 1;
    if (p < kSink) {
      uint16_t* sink = (is_v ? d.sink_v : d.sink_k) + (static_cast<size_t>(b) * hkv + kvh) * kSink * kDim;
      sink[p * kDim + k] = val;
    } else {
      recent[((p - kSink) & (kRecent - 1)) * kDim + k] = val;
    }
  }
}

// Runtime-G dispatch of demote_unit.
template <int NT = kDim>
__device__ __forceinline__ void demote_unit_g(int group, const DemoteStep& d, int kvh, int b, bool is_v, int k,
                                              QuantSmem<1>& sm) {
  if (group == 32) demote_unit<32, NT>(d, kvh, b, is_v, k, sm);
  else if (group == 64) demote_unit<64, NT>(d, kvh, b, is_v, k, sm);
  else demote_unit<128, NT>(d, kvh, b, is_v, k, sm);
}

}  // namespace
}  // namespace oscar
