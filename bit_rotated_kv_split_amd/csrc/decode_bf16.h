// Decode attention over the bf16 sink and recent tokens (page
// "超越TurboQuant：Together AI把2-bit KV Cache推向真实服务", section
// "OSCAR的另一个关键点是": a bf16 kernel handles sink and recent, with the
// unrotated query).  Five 64-slot chunks per (request, KV head): the sink,
// then the recent ring in quarters; one wave each, each writing its own
// partial (output, natural-log LSE) into the decode workspace.
//   q . k: lane = token, its 256-byte key row in sixteen 16-byte loads;
//   p . v: lane = (8-channel group, token residue mod 4), 16-byte loads
//          coalesced along each value row, reduced over the residues.
// Rows are read a quarter at a time (four 16-byte loads in flight per lane)
// to keep the register count low.
#pragma once

#include <math.h>

#include "oscar_device.h"
#include "oscar_internal.h"

namespace oscar {

struct Bf16Params {
  const uint16_t* q;
  const uint16_t* sink_k;
  const uint16_t* sink_v;
  const uint16_t* recent_k;
  const uint16_t* recent_v;
  const int32_t* seq_lens;
  float* po;            // [B][Hq][5][128]
  float* plse;          // [B][Hq][5]
  int32_t hkv;
  int32_t hq;
};

template <int GQ>
struct Bf16Smem {
  float q[GQ][kDim];
  float p[GQ][kPage];
};

inline Bf16Params make_bf16_params(const DecodeArgs& a) {
  Bf16Params p;
  p.q = a.q;
  p.sink_k = a.cache->sink_k;
  p.sink_v = a.cache->sink_v;
  p.recent_k = a.cache->recent_k;
  p.recent_v = a.cache->recent_v;
  p.seq_lens = a.cache->seq_lens;
  p.po = reinterpret_cast<float*>(a.ws + a.lay.off_bo);
  p.plse = reinterpret_cast<float*>(a.ws + a.lay.off_blse);
  p.hkv = a.dims->num_kv_heads;
  p.hq = a.dims->num_q_heads;
  return p;
}

// One chunk for query heads h_lo .. h_lo + nh - 1 (nh = min(GQ, gq - h_lo))
// of the gq-head group of KV head kvh, request b.  Called by a whole 64-lane
// wave.
template <int GQ>
__device__ __forceinline__ void bf16_chunk(const Bf16Params& a, int gq, int h_lo, int chunk, int kvh, int b,
                                           Bf16Smem<GQ>& sm) {
  const int lane = threadIdx.x & 63;
  const int nh = min(GQ, gq - h_lo);
  const int L = a.seq_lens[b];
  const int n_sink = min(L, kSink);
  const int n_recent = min(max(L - kSink, 0), kRecent);
  const int n_valid = chunk == 0 ? n_sink : min(max(n_recent - (chunk - 1) * kPage, 0), kPage);
  const size_t head0 = static_cast<size_t>(b) * a.hq + static_cast<size_t>(kvh) * gq + h_lo;
  if (n_valid == 0) {   // uniform across the wave
    for (int i = lane; i < nh * kDim; i += 64)
      a.po[((head0 + i / kDim) * kBf16Parts + chunk) * kDim + i % kDim] = 0.f;
    if (lane < nh) a.plse[(head0 + lane) * kBf16Parts + chunk] = -INFINITY;
    return;
  }
  for (int i = lane; i < GQ * kDim; i += 64)
    sm.q[i / kDim][i % kDim] = i / kDim < nh ? bf16_to_f32(a.q[head0 * kDim + i]) * kScoreScaleLog2 : 0.f;
  const size_t kv0 = static_cast<size_t>(b) * a.hkv + kvh;
  const uint16_t* kb = chunk == 0 ? a.sink_k + kv0 * kSink * kDim
                                  : a.recent_k + (kv0 * kRecent + (chunk - 1) * kPage) * kDim;
  const uint16_t* vb = chunk == 0 ? a.sink_v + kv0 * kSink * kDim
                                  : a.recent_v + (kv0 * kRecent + (chunk - 1) * kPage) * kDim;
  const bool valid = lane < n_valid;
  // key row of this lane's token (a valid row is read either way), a
  // quarter (64 bytes) at a time: the chunk runs inside the matrix-core
  // history kernel, whose register budget it must not raise
  float sc[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) sc[h] = 0.f;
  const uint4* row = reinterpret_cast<const uint4*>(kb + (valid ? lane : 0) * kDim);
#pragma unroll 1
  for (int qt = 0; qt < 4; ++qt) {
    uint4 krow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) krow[i] = row[4 * qt + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ws[4] = {krow[i].x, krow[i].y, krow[i].z, krow[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(ws[j] << 16);
        const float hi = __uint_as_float(ws[j] & 0xFFFF0000u);
        const int ch = (4 * qt + i) * 8 + 2 * j;
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
          sc[h] = __builtin_fmaf(sm.q[h][ch], lo, sc[h]);
          sc[h] = __builtin_fmaf(sm.q[h][ch + 1], hi, sc[h]);
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float mx[GQ], lsum[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const float s = valid ? sc[h] : -INFINITY;
    mx[h] = wave_max(s);
    const float pr = valid ? exp2f(s - mx[h]) : 0.f;
    lsum[h] = wave_sum(pr);
    sm.p[h][lane] = pr;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int cg = lane & 15, res = lane >> 4;
  float acc[GQ][8];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  // value rows a quarter (four tokens per lane) at a time, as for the keys
#pragma unroll 1
  for (int qt = 0; qt < 4; ++qt) {
    uint4 vrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = res + 4 * (4 * qt + i);
      vrow[i] = *reinterpret_cast<const uint4*>(vb + (t < n_valid ? t : 0) * kDim + cg * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = res + 4 * (4 * qt + i);
      const uint32_t ws[4] = {vrow[i].x, vrow[i].y, vrow[i].z, vrow[i].w};
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float pt = t < n_valid ? sm.p[h][t] : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[h][2 * j] = __builtin_fmaf(pt, __uint_as_float(ws[j] << 16), acc[h][2 * j]);
          acc[h][2 * j + 1] = __builtin_fmaf(pt, __uint_as_float(ws[j] & 0xFFFF0000u), acc[h][2 * j + 1]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const float inv = 1.f / lsum[h];
    const size_t pidx = (head0 + h) * kBf16Parts + chunk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (res == 0 && h < nh) a.po[pidx * kDim + cg * 8 + e] = v * inv;
    }
    if (lane == 0 && h < nh) a.plse[pidx] = (mx[h] + log2f(lsum[h])) * kLn2;
  }
}

}  // namespace oscar
