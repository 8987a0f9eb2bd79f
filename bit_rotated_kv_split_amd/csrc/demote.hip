// Demotion: rotate -> clip -> quantize -> pack of bf16 tokens into INT2
// history pages (page "超越TurboQuant：Together AI把2-bit KV Cache推向真实服务",
// section "OSCAR的另一个关键点是"), in two launch shapes:
//   * demote_kernel: one decode step, the oldest recent token of every
//     (request, KV head), followed by the append of the new token into the
//     freed slot;
//   * fill_kernel: up to 16 consecutive history tokens per workgroup (all
//     inside one 16-token value word), for filling history in bulk.
// Both run the same per-token arithmetic (quantize_tokens, demote_device.h);
// the decode prologue (decode.hip) runs demote_unit as well.
//
// A workgroup has 128 threads, thread k owning stored channel k.  The
// rotation is a 128x128 GEMV per token with the rotation row read once per
// workgroup and reused across its tokens.  A bf16 x float32 product is exact
// in float64, so the GEMV accumulates in float64 and rounds once to float32:
// the stored value is the rounded exact dot product except where the
// float64 rounding of the sum lands within ~2^-22 ulp of a float32 tie.
// Quantization uses IEEE float32 subtraction and division (no fast-math)
// and round-half-even, so the codes and the bf16 scale/zero are a
// deterministic function of the rotated values (for the Lloyd-Max codebook
// up to the summation order of the float64 group mean and variance).
#include "demote_device.h"

namespace oscar {
namespace {

template <int G>
__global__ void __launch_bounds__(128)
demote_kernel(DemoteStep d) {
  __shared__ QuantSmem<1> sm;
  demote_unit<G>(d, blockIdx.x, blockIdx.y, blockIdx.z != 0, threadIdx.x, sm);
}

template <int G>
__global__ void __launch_bounds__(128)
fill_kernel(DemoteArgs kk, DemoteArgs vv, int32_t request, int32_t hist_begin, int32_t n_tokens,
            const uint16_t* __restrict__ k_tokens, const uint16_t* __restrict__ v_tokens) {
  __shared__ QuantSmem<kMaxChunk> sm;
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
                                a.clip + kvh * kDim, k, a.codebook, a.thr);
  const int phys = a.page_table[static_cast<size_t>(request) * a.max_pages + (j0 >> 6)];
  uint8_t* blk = a.pages + (static_cast<size_t>(phys) * hkv + kvh) * block_bytes(G);
  store_tokens<G, kMaxChunk>(sm, nt, blk, j0 & 63, is_v, k);
}

// Dequantized history values of one (request, KV head, K or V) for up to 64
// consecutive history indices starting at hist_begin + 64 * blockIdx.x
// (128 threads, thread = channel).  Uniform codebook: one float32 rounding
// of code * scale + zero; Lloyd-Max: zero + scale * level in float64 (the
// product and the sum each rounded, not fused), then rounded to float32.
__global__ void __launch_bounds__(128)
read_history_kernel(const uint8_t* __restrict__ pages, const int32_t* __restrict__ page_table, int32_t max_pages,
                    int32_t hkv, int32_t group, int32_t codebook, Codebook cb, int32_t request, int32_t hist_begin,
                    int32_t n_tokens, float* __restrict__ k_out, float* __restrict__ v_out) {
  const int kvh = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int c = threadIdx.x;
  const int ng = kDim / group, gi = c / group;
  const int t0 = 64 * blockIdx.x;
  const int t1 = min(t0 + 64, n_tokens);
  float* out = is_v ? v_out : k_out;
  for (int t = t0; t < t1; ++t) {
    const int j = hist_begin + t;
    const int phys = page_table[static_cast<size_t>(request) * max_pages + (j >> 6)];
    const uint8_t* blk = pages + (static_cast<size_t>(phys) * hkv + kvh) * block_bytes(group);
    const uint32_t* words = reinterpret_cast<const uint32_t*>(blk);
    const int slot = j & 63;
    uint32_t code;
    if (!is_v) code = ((words[(c >> 4) * 64 + qk_order(slot)] ^ kTopFieldFlip) >> (2 * (c & 15))) & 3u;
    else code = ((words[512 + v_word_index(c, slot >> 4)] ^ kTopFieldFlip) >> (2 * (slot & 15))) & 3u;
    const uint16_t* sz = reinterpret_cast<const uint16_t*>(blk + kCodesBytes + (is_v ? kPage * ng * 4 : 0)) +
                         (qk_order(slot) * ng + gi) * 2;
    const float s = bf16_to_f32(sz[0]), z = bf16_to_f32(sz[1]);
    float y;
    if (codebook == OSCAR_CODEBOOK_LLOYD_MAX)
      y = static_cast<float>(__dadd_rn(static_cast<double>(z),
                                       __dmul_rn(static_cast<double>(s), static_cast<double>(cb.lev[code]))));
    else
      y = __builtin_fmaf(static_cast<float>(code), s, z);   // code * s is exact: one rounding
    out[(static_cast<size_t>(t) * hkv + kvh) * kDim + c] = y;
  }
}

DemoteArgs make_args(const oscar_dims& d, const oscar_cache& c, const float* r, const float* clip) {
  DemoteArgs a;
  a.r = r;
  a.clip = clip;
  a.pages = c.pages;
  a.page_table = c.page_table;
  a.max_pages = c.max_pages_per_req;
  a.hkv = d.num_kv_heads;
  a.codebook = d.codebook;
  a.thr = codebook_of(d.codebook)->thr[2];
  return a;
}

}  // namespace

DemoteStep make_demote_step(const oscar_dims& d, const oscar_rotation& rot, const oscar_cache& c,
                            const uint16_t* k_new, const uint16_t* v_new) {
  DemoteStep st;
  st.kk = make_args(d, c, rot.r_k, rot.clip_k);
  st.vv = make_args(d, c, rot.r_v, rot.clip_v);
  st.seq_lens = c.seq_lens;
  st.sink_k = c.sink_k;
  st.sink_v = c.sink_v;
  st.recent_k = c.recent_k;
  st.recent_v = c.recent_v;
  st.k_new = k_new;
  st.v_new = v_new;
  return st;
}

hipError_t launch_demote(const oscar_dims& d, const oscar_rotation& rot, const oscar_cache& c,
                         const uint16_t* k_new, const uint16_t* v_new, hipStream_t s) {
  const DemoteStep st = make_demote_step(d, rot, c, k_new, v_new);
  const dim3 grid(d.num_kv_heads, c.batch, 2);
  switch (d.group_size) {
    case 32: demote_kernel<32><<<grid, 128, 0, s>>>(st); break;
    case 64: demote_kernel<64><<<grid, 128, 0, s>>>(st); break;
    default: demote_kernel<128><<<grid, 128, 0, s>>>(st); break;
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

hipError_t launch_read_history(const oscar_dims& d, const oscar_cache& c, int32_t request, int32_t hist_begin,
                               int32_t n_tokens, float* k_out, float* v_out, hipStream_t s) {
  const dim3 grid((n_tokens + 63) / 64, d.num_kv_heads, 2);
  read_history_kernel<<<grid, 128, 0, s>>>(c.pages, c.page_table, c.max_pages_per_req, d.num_kv_heads, d.group_size,
                                           d.codebook, *codebook_of(d.codebook), request, hist_begin, n_tokens, k_out,
                                           v_out);
  return hipGetLastError();
}

}  // namespace oscar
