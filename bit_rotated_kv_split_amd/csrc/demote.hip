// Demotion: rotate -> clip -> quantize -> pack of bf16 tokens into INT2
// history pages (page "超越TurboQuant：Together AI把2-bit KV Cache推向真实服务",
// section "OSCAR的另一个关键点是"), in two launch shapes:
//   * demote_kernel: one decode step, the oldest recent token of every
//     (request, KV head), followed by the append of the new token into the
//     freed slot;
//   * fill_kernel: up to 16 consecutive history tokens per workgroup (all
//     inside one 16-token value word), for filling history in bulk.
// Both run the same per-token arithmetic (quantize_tokens below).
//
// A workgroup has 128 threads, thread k owning stored channel k.  The
// rotation is a 128x128 GEMV per token with the rotation row read once per
// workgroup and reused across its tokens.  A bf16 x float32 product is exact
// in float64, so the GEMV accumulates in float64 and rounds once to float32:
// the stored value is the rounded exact dot product except where the
// float64 rounding of the sum lands within ~2^-22 ulp of a float32 tie.
// Quantization uses IEEE float32 subtraction and division (no fast-math)
// and round-half-even, so the codes and the bf16 scale/zero are a
// deterministic function of the rotated values.
#include "oscar_device.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr int kMaxChunk = 16;

template <int G, int NT>
struct QuantSmem {
  static constexpr int NG = kDim / G;
  float x[NT][kDim];
  float y[NT][kDim];
  float scale[NT][NG];
  float zero[NT][NG];
  uint8_t code[NT][kDim];
};

// Rotate, clip and quantize nt (<= NT) tokens held in sm.x.  All 128 threads
// of the workgroup must call it.  Leaves codes, scale and zero in shared memory.
template <int G, int NT>
__device__ void quantize_tokens(QuantSmem<G, NT>& sm, int nt, const float* __restrict__ r,
                                const float* __restrict__ clipv) {
  constexpr int WG = G < 64 ? G : 64;   // group lanes inside one wave
  const int k = threadIdx.x, lane = k & 63, wave = k >> 6;
  __shared__ float xw[2][NT][2];        // per-wave (min, max) when a group spans both waves
  double acc[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = 0.0;
  if constexpr (NT == 1) {
    // one token: every load of the rotation column in flight at once
    float rv[kDim];
#pragma unroll
    for (int i = 0; i < kDim; ++i) rv[i] = r[i * kDim + k];
#pragma unroll
    for (int i = 0; i < kDim; ++i)
      acc[0][i & 3] = fma(static_cast<double>(sm.x[0][i]), static_cast<double>(rv[i]), acc[0][i & 3]);
  } else {
    for (int i = 0; i < kDim; i += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double rik = static_cast<double>(r[(i + u) * kDim + k]);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][u] = fma(static_cast<double>(sm.x[t][i + u]), rik, acc[t][u]);
      }
    }
  }
  const float c = clipv[k];
  float y[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const double sum = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
    y[t] = fminf(fmaxf(static_cast<float>(sum), -c), c);
    sm.y[t][k] = y[t];
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
  const int gi = k / G;
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
__device__ void store_tokens(const QuantSmem<G, NT>& sm, int nt, uint8_t* __restrict__ blk,
                             int slot0, bool is_v) {
  constexpr int NG = kDim / G;
  const int k = threadIdx.x;
  uint32_t* words = reinterpret_cast<uint32_t*>(blk);
  if (!is_v) {
    for (int job = k; job < nt * 8; job += kDim) {
      const int t = job >> 3, d = job & 7;
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) w |= static_cast<uint32_t>(sm.code[t][16 * d + i]) << (2 * i);
      words[d * 64 + qk_order(slot0 + t)] = w;
    }
  } else {
    // channel k: one value word holds slots 16w..16w+15 of this channel
    const int w = slot0 >> 4;
    uint32_t bits = 0, mask = 0;
    for (int t = 0; t < nt; ++t) {
      const int sh = 2 * ((slot0 + t) & 15);
      bits |= static_cast<uint32_t>(sm.code[t][k]) << sh;
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

template <int G>
__global__ void __launch_bounds__(128)
demote_kernel(DemoteArgs kk, DemoteArgs vv, const int32_t* __restrict__ seq_lens,
              uint16_t* __restrict__ sink_k, uint16_t* __restrict__ sink_v,
              uint16_t* __restrict__ recent_k, uint16_t* __restrict__ recent_v,
              const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new) {
  __shared__ QuantSmem<G, 1> sm;
  const int kvh = blockIdx.x, b = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const DemoteArgs& a = is_v ? vv : kk;
  const int hkv = a.hkv;
  const int k = threadIdx.x;
  const int L = seq_lens[b];
  uint16_t* recent = (is_v ? recent_v : recent_k) + (static_cast<size_t>(b) * hkv + kvh) * kRecent * kDim;
  if (L > kBf16Tokens) {
    const int j = L - kBf16Tokens - 1;            // history index of position L-257
    const int ring = (L - 1 - kSink) & (kRecent - 1);
    sm.x[0][k] = bf16_to_f32(recent[ring * kDim + k]);
    __syncthreads();
    quantize_tokens<G, 1>(sm, 1, a.r + static_cast<size_t>(kvh) * kDim * kDim,
                          a.clip + kvh * kDim);
    const int phys = a.page_table[static_cast<size_t>(b) * a.max_pages + (j >> 6)];
    uint8_t* blk = a.pages + (static_cast<size_t>(phys) * hkv + kvh) * block_bytes(G);
    store_tokens<G, 1>(sm, 1, blk, j & 63, is_v);
  }
  const uint16_t* src = is_v ? v_new : k_new;
  if (src != nullptr && L >= 1) {
    const int p = L - 1;
    const uint16_t val = src[(static_cast<size_t>(b) * hkv + kvh) * kDim + k];
    if (p < kSink) {
      uint16_t* sink = (is_v ? sink_v : sink_k) + (static_cast<size_t>(b) * hkv + kvh) * kSink * kDim;
      sink[p * kDim + k] = val;
    } else {
      recent[((p - kSink) & (kRecent - 1)) * kDim + k] = val;
    }
  }
}

template <int G>
__global__ void __launch_bounds__(128)
fill_kernel(DemoteArgs kk, DemoteArgs vv, int32_t request, int32_t hist_begin, int32_t n_tokens,
            const uint16_t* __restrict__ k_tokens, const uint16_t* __restrict__ v_tokens) {
  __shared__ QuantSmem<G, kMaxChunk> sm;
  const int kvh = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const DemoteArgs& a = is_v ? vv : kk;
  const int hkv = a.hkv;
  const int k = threadIdx.x;
  const int hist_end = hist_begin + n_tokens;
  const int c0 = (hist_begin & ~(kMaxChunk - 1)) + kMaxChunk * blockIdx.x;
  const int j0 = max(c0, hist_begin);
  const int j1 = min(c0 + kMaxChunk, hist_end);
  const int nt = j1 - j0;
  if (nt <= 0) return;   // uniform across the workgroup
  const uint16_t* src = is_v ? v_tokens : k_tokens;
  for (int t = 0; t < nt; ++t)
    sm.x[t][k] = bf16_to_f32(src[(static_cast<size_t>(j0 - hist_begin + t) * hkv + kvh) * kDim + k]);
  for (int t = nt; t < kMaxChunk; ++t) sm.x[t][k] = 0.f;
  __syncthreads();
  quantize_tokens<G, kMaxChunk>(sm, nt, a.r + static_cast<size_t>(kvh) * kDim * kDim,
                                a.clip + kvh * kDim);
  const int phys = a.page_table[static_cast<size_t>(request) * a.max_pages + (j0 >> 6)];
  uint8_t* blk = a.pages + (static_cast<size_t>(phys) * hkv + kvh) * block_bytes(G);
  store_tokens<G, kMaxChunk>(sm, nt, blk, j0 & 63, is_v);
}

DemoteArgs make_args(const oscar_dims& d, const oscar_cache& c, const float* r, const float* clip) {
  DemoteArgs a;
  a.r = r;
  a.clip = clip;
  a.pages = c.pages;
  a.page_table = c.page_table;
  a.max_pages = c.max_pages_per_req;
  a.hkv = d.num_kv_heads;
  return a;
}

}  // namespace

hipError_t launch_demote(const oscar_dims& d, const oscar_rotation& rot, const oscar_cache& c,
                         const uint16_t* k_new, const uint16_t* v_new, hipStream_t s) {
  const DemoteArgs kk = make_args(d, c, rot.r_k, rot.clip_k);
  const DemoteArgs vv = make_args(d, c, rot.r_v, rot.clip_v);
  const dim3 grid(d.num_kv_heads, c.batch, 2);
  switch (d.group_size) {
    case 32:
      demote_kernel<32><<<grid, 128, 0, s>>>(kk, vv, c.seq_lens, c.sink_k, c.sink_v, c.recent_k,
                                             c.recent_v, k_new, v_new);
      break;
    case 64:
      demote_kernel<64><<<grid, 128, 0, s>>>(kk, vv, c.seq_lens, c.sink_k, c.sink_v, c.recent_k,
                                             c.recent_v, k_new, v_new);
      break;
    default:
      demote_kernel<128><<<grid, 128, 0, s>>>(kk, vv, c.seq_lens, c.sink_k, c.sink_v, c.recent_k,
                                              c.recent_v, k_new, v_new);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_fill(const oscar_dims& d, const oscar_rotation& rot, const oscar_cache& c,
                       int32_t request, int32_t hist_begin, int32_t n_tokens,
                       const uint16_t* k_tokens, const uint16_t* v_tokens, hipStream_t s) {
  const DemoteArgs kk = make_args(d, c, rot.r_k, rot.clip_k);
  const DemoteArgs vv = make_args(d, c, rot.r_v, rot.clip_v);
  const int first = hist_begin & ~(kMaxChunk - 1);
  const int chunks = (hist_begin + n_tokens - first + kMaxChunk - 1) / kMaxChunk;
  const dim3 grid(chunks, d.num_kv_heads, 2);
  switch (d.group_size) {
    case 32:
      fill_kernel<32><<<grid, 128, 0, s>>>(kk, vv, request, hist_begin, n_tokens, k_tokens, v_tokens);
      break;
    case 64:
      fill_kernel<64><<<grid, 128, 0, s>>>(kk, vv, request, hist_begin, n_tokens, k_tokens, v_tokens);
      break;
    default:
      fill_kernel<128><<<grid, 128, 0, s>>>(kk, vv, request, hist_begin, n_tokens, k_tokens, v_tokens);
      break;
  }
  return hipGetLastError();
}

}  // namespace oscar
