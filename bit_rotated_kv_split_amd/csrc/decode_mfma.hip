// Matrix-core history kernel: split-K decode attention over INT2 history
// pages (page "超越TurboQuant：Together AI把2-bit KV Cache推向真实服务",
// section "OSCAR的另一个关键点是": unpack, scale/zero dequantization and
// float accumulation of the INT2 history), built on v_mfma_i32_16x16x64_i8.
//
// The vector-ALU form needs ~1000 fp32 FMAs per history token and KV head
// (q.k and p.v for four query heads), twice what the vector ALU can retire
// while HBM streams the 72 bytes that token costs.  Both contractions are
// exact integer products here:
//   q . code   A = the rotated query as 4-digit signed base-256 fixed point
//              (rows = head x digit), B = 2-bit codes as int8;
//   P' . code  A = p * value-scale per token as 4 signed base-256 digits
//              (rows = head x digit), B = value codes as int8.
// A word of sixteen 2-bit codes gives the four int8 operand registers as
// w & 0x03030303 << 2j, four operations: the code times 4^j masked in place
// for j = 0, 1, 2, and for j = 3, whose codes are stored XOR 2, the signed
// byte 64 (code - 2).  The A operand of those slots carries the matching
// 4^-j (query digits are rounded on that grid, P' digits are computed from
// floats and lose nothing).  The -2 of the j = 3 slots adds -128 times the
// digit to every product: for q . code the accumulators start from +128
// times the query's j = 3 digit sums (one set of products per wave, before
// the pages); for P' . code the same sums of the P' digits are accumulated
// per page by one more product against a constant operand, and added back
// when the accumulators are read.
//
// Softmax bookkeeping is amortised over pages.  Each head keeps a reference
// maximum m and a fixed-point unit u; tokens use p = 2^(score - m) and
// digits of p * scale / u, so the P' . code products of many pages add up
// exactly in the MFMA's int32 accumulator, and l = sum p and the zero-point
// sum p * zero stay per-lane partial sums.  A head "re-bases" (its int32
// accumulator is folded into float, everything rescaled by 2^(m_old - m_new),
// and a new unit taken from the current page) only when a score exceeds m by
// more than kSlack or a value would overflow the digits; that branch is
// uniform across the wave and rare once the first page has set m.
//
// The digits of P' are rounded with error diffusion: each lane carries the
// part of its last weight that rounding dropped into its next one.  Plain
// rounding would lose the many weights far below the unit (the unit follows
// the largest weight) while the zero-point sum and l keep them, which biases
// the output along the dominant value direction; with the carry the
// rounded weights of a lane add up to the exact ones within half a unit.
//
// The Lloyd-Max codebook (levels -hi, -lo, lo, hi for codes 0..3) splits a
// code c = 2 b1 + b0 into bit planes: level(c) = -hi + (hi - lo) c +
// (3 lo - hi) b1.  The c plane is the uniform kernel's operand; the b1 plane
// is the same masked word ANDed down to its high bits (2 b1 4^j).  For keys
// the plane goes against a second query operand holding q (3 lo - hi) /
// (2 (hi - lo)), accumulating into the same result; for values it has its
// own accumulators against the same P' operand.  The -hi term joins the zero
// point (zero - hi * scale per token and group).
//
// A workgroup owns (history split, KV head, request) with one wave per four
// query heads (two waves for eight-head groups), and five more workgroups
// per (KV head, request) run the bf16 sink/recent chunks (decode_bf16.h)
// alongside the history splits.  Per 64-token page a lane loads 4 x 16 B of
// codes and the scale/zero entries of its tokens (the page layout puts each
// lane's MFMA operands in one 16-byte load); the loads of the next BUF-1
// pages are in flight while a page is processed (register buffers, no
// copies; BUF per instantiation in HistShape).  Query heads are handled in
// blocks of four (16 MFMA rows = 4 heads x 4 digit rows).
#include <math.h>

#include <hip/hip_ext.h>

#include "decode_bf16.h"
#include "oscar_device.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// Launch-shape knobs (compile-time): register page buffers per wave (2 or 3)
// and the waves per SIMD the register budget is sized for.
#ifndef OSCAR_HIST_BUFFERS
#define OSCAR_HIST_BUFFERS 2
#endif
// software-pipelined page loop (value half of page p-1 before the score
// half of page p) for G >= 64: 32 x 100K Lloyd-Max 325.5 -> 320.9 us,
// 1 x 100K 20.9 -> 20.3 us, G = 128 and 64 about 0.3 % faster; at G = 32
// it measured 1 % slower and is not used there
#ifndef OSCAR_HIST_PIPE
#define OSCAR_HIST_PIPE 1
#endif
#ifndef OSCAR_HIST_MIN_WAVES
#define OSCAR_HIST_MIN_WAVES 2
#endif
// the Lloyd-Max form holds a second set of value accumulators (two
// buffers measured 3 % faster than three)
#ifndef OSCAR_HIST_BUFFERS_LM
#define OSCAR_HIST_BUFFERS_LM 2
#endif
#ifndef OSCAR_HIST_MIN_WAVES_LM
#define OSCAR_HIST_MIN_WAVES_LM OSCAR_HIST_MIN_WAVES
#endif
// G = 32 pages carry four scale/zero pairs per token and K/V (48 VGPRs a
// buffer); its Lloyd-Max form keeps one buffer (two spill)
#ifndef OSCAR_HIST_BUFFERS_32
#define OSCAR_HIST_BUFFERS_32 2
#endif

constexpr float kSlack = 2.0f;                 // log2 headroom of p above 1 before re-basing
constexpr float kHeadroom = 8.0f;              // 2^kSlack times 2x room for larger value scales
// P' digits: x < 2^31 - 2^24.  With y = x + 0x808080 (below 2^31), the
// bytes of y are x's four signed base-256 digits, the three low ones plus
// 128 (their top bits flipped before the word is stored) and the top one as
// it is.  (The offset is added to the converted integer: added to the float
// weight it would round away the fraction that the carry keeps.)
constexpr float kDigitLimit = 2130706432.0f;
constexpr uint32_t kDigitOffset = 0x808080u;
constexpr uint32_t kLowDigitFlip = 0x00808080u;   // bytes 0..2 of a token's digit word
constexpr float kDigitUnitMax = 2147483648.0f; // the unit puts a page's largest weight at 2^28
// Pages a head's int32 accumulators may take between folds: a page adds at
// most 64 * 128 * 128 to a digit row (the j = 3 operand bytes reach -128).
constexpr int kFoldPages = 2047;

// Codes at positions 4b+j of a stored 16-code word -> byte b of result j:
// the code times 4^j for j < 3, and 64 (code - 2) for j = 3 (stored XOR 2).
__device__ __forceinline__ v4i unpack16(uint32_t w) {
  v4i r;
  r.x = static_cast<int>(w & 0x03030303u);
  r.y = static_cast<int>(w & 0x0C0C0C0Cu);
  r.z = static_cast<int>(w & 0x30303030u);
  r.w = static_cast<int>(w & 0xC0C0C0C0u);
  return r;
}

// High bits of the masked codes of unpack16: 2 b1 4^j in place of c 4^j,
// and for j = 3 (stored bit 7 = not b1) the signed byte 64 (2 b1 - 2).
__device__ __forceinline__ v4i high_bits(const v4i& r) {
  v4i h;
  h.x = r.x & 0x02020202;
  h.y = r.y & 0x08080808;
  h.z = r.z & 0x20202020;
  h.w = r.w & static_cast<int>(0x80808080u);
  return h;
}

// Operand with +64 in every j = 3 slot: a product against it sums the A
// operand's j = 3 digits (times 64) along each row.
__device__ __forceinline__ v4i j3_ones() {
  v4i r;
  r.x = 0;
  r.y = 0;
  r.z = 0;
  r.w = 0x40404040;
  return r;
}

// value of the signed base-256 digit rows of q . code: a row sums 128
// products of a digit (|d| <= 128) and a byte (|b| <= 128) plus its start
// value, so both two-row integer sums fit in int32
__device__ __forceinline__ float q_digits(const v4i& d) {
  const int lo = d.x + (d.y << 8);
  const int hi = d.z + (d.w << 8);
  return __builtin_fmaf(65536.f, static_cast<float>(hi), static_cast<float>(lo));
}

// value of the signed base-256 digit rows of P' . code (accumulated)
__device__ __forceinline__ float p_digits(const v4i& d) {
  return static_cast<float>(d.x) + 256.f * static_cast<float>(d.y) + 65536.f * static_cast<float>(d.z) +
         16777216.f * static_cast<float>(d.w);
}

// 8-byte read from LDS transposed across each 16-lane group
// (ds_read_b64_tr_b8): lane 16 g + 8 h + b receives, as its byte i, byte b
// of the 8 bytes that lane 16 g + 2 i + h addressed (checked lane by lane on
// the device with permuted addresses).
typedef int v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2i lds_read_tr8(const int32_t* p) {
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  // a generic address of LDS data holds the LDS offset in its low 32 bits
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (lds_v2i*)static_cast<size_t>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p))));
}

// Reductions over the 16 lanes of a DPP row (lanes 16r .. 16r+15).
template <typename Op>
__device__ __forceinline__ float row_reduce(float v, Op op) {
  int x = __float_as_int(v);
  x = __float_as_int(op(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false))));
  x = __float_as_int(op(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false))));
  x = __float_as_int(op(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false))));
  x = __float_as_int(op(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false))));
  return __int_as_float(x);
}

// float64 sum over the 16 lanes of a DPP row.
template <int CTRL>
__device__ __forceinline__ double dpp_add_f64(double v) {
  const int lo = __double2loint(v), hi = __double2hiint(v);
  const int plo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  const int phi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
  return v + __hiloint2double(phi, plo);
}
__device__ __forceinline__ double row_sum_f64(double v) {
  v = dpp_add_f64<0xB1>(v);
  v = dpp_add_f64<0x4E>(v);
  v = dpp_add_f64<0x141>(v);
  return dpp_add_f64<0x140>(v);
}

struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};

struct MfmaParams {
  const uint8_t* pages;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const uint8_t* qpack;
  const float* qsum;
  const int32_t* sched;   // split table: [0] = count, then {request, first page, end page}
  float* po;              // [slots][Hq][128]
  float* plse;            // [slots][Hq]
  int32_t max_pages;
  int32_t hkv;
  int32_t hq;
  int32_t gq;
  int32_t slots;          // history workgroups per KV head in the grid
  float lm_hi;            // Lloyd-Max: the outer level hi
  float lm_ka;            // hi - lo: weight of the code plane
  float lm_kb;            // (3 lo - hi) / 2: weight of the 2 b1 plane
  Bf16Params bf;          // the bf16 sink/recent chunks, run as extra workgroups
  unsigned long long* clk;   // timing hook or nullptr: workgroup 0's clock counters
};

template <int G>
struct PageRegs {
  static constexpr int NG = kDim / G;
  v4i kw[2];              // key words: half hf, word m -> token tau(m, n), word d = 4 hf + lane group
  v4i vw[2];              // value words: load r, word m -> channel block 4 r + m
  uint32_t ksz[4 * NG];   // (scale, zero) bf16 pairs of tokens tau(m, n), [m][group]
  uint32_t vsz[4 * NG];
};

// 16-byte load through a buffer resource: scalar base, per-lane 32-bit
// offset, so a page costs no vector address arithmetic.  STREAM sets the
// non-temporal policy bit (aux 2).  A one-wave kernel reads its code words
// once, and with non-temporal loads HBM streams them faster (32 x 100K,
// G = 128: 326 -> 283 us; 16 x 128K: 218 -> 190 us).  The two-wave kernels
// read every page twice, the second wave mostly from cache, and keep
// ordinary loads (non-temporal: 284 -> 323 us on the ragged GQA-8 batch).
template <bool STREAM>
__device__ __forceinline__ v4i load16r(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, STREAM ? 2 : 0));
}

// Raw-buffer resource word 3 for gfx9-family (untyped 32-bit data)
constexpr int kRsrcWord3 = 0x00020000;

// STREAM_SZ: the scale/zero entries non-temporal too (the kernel decides
// per instantiation).  blk is wave-uniform; the resource covers exactly the
// block (a read past it would return 0; none is made).
template <int G, bool STREAM, bool STREAM_SZ>
__device__ __forceinline__ void load_page(PageRegs<G>& r, const uint8_t* __restrict__ blk, int lane) {
  constexpr int NG = kDim / G;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), 0, block_bytes(G), kRsrcWord3);
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
  const uint32_t so = static_cast<uint32_t>(kCodesBytes) + static_cast<uint32_t>(lane & 15) * (16u * NG);
  r.kw[0] = load16r<STREAM>(rs, lo, 0);
  r.kw[1] = load16r<STREAM>(rs, lo, 1024);
  r.vw[0] = load16r<STREAM>(rs, lo, 2048);
  r.vw[1] = load16r<STREAM>(rs, lo, 3072);
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const v4i a = load16r<STREAM_SZ>(rs, so, 16 * i);
    const v4i b = load16r<STREAM_SZ>(rs, so, kPage * NG * 4 + 16 * i);
    r.ksz[4 * i + 0] = a.x; r.ksz[4 * i + 1] = a.y; r.ksz[4 * i + 2] = a.z; r.ksz[4 * i + 3] = a.w;
    r.vsz[4 * i + 0] = b.x; r.vsz[4 * i + 1] = b.y; r.vsz[4 * i + 2] = b.z; r.vsz[4 * i + 3] = b.w;
  }
}

template <int NHB, int G>
struct WaveState {
  static constexpr int NG = kDim / G;
  v4i qa[NHB][2];          // query digit operands
  v4i qb[NHB][2];          // Lloyd-Max only: the same for q times the high-bit weight ratio
  // G = 32 only: the operands of each half masked to one of its two groups
  // (lane groups 2 sub, 2 sub + 1 hold the group's 32 channels)
  v4i qam[NHB][2][2];
  v4i qbm[NHB][2][2];
  float qs[NHB];           // query fixed-point unit of this lane's head (1 for an all-zero query)
  float qz[NHB][NG];       // per-group query sums / qs (zero-point term of the score / qs)
  float m_ref[NHB];        // reference maximum (log2 units)
  float unit[NHB][NG];     // P' fixed-point unit
  float inv[NHB][NG];      // 4^-j / unit for this lane's token residue j
  // the j = 3 P' sums are counted by an extra product per group for G >= 64;
  // at G = 32 (four groups, the register budget is spent) the correction
  // joins the zero-point sums instead (zc)
  static constexpr bool kDcorr = NG <= 2;
  v4i kc[NHB][NG];         // q . code start values: 128 x the query's j = 3 digit sums per product
  v4i dcorr[NHB][kDcorr ? NG : 1];   // 64 x the j = 3 P' digit sums per group (added back x 2 when read)
  float zc;                // this lane's value-zero coefficient of the scale: -hi (Lloyd-Max), plus
                           // the j = 3 correction when !kDcorr
  v4i dacc[NHB][8];        // int32 digit accumulators of P' . code, channel block cb
  v4i dacc1[NHB][8];       // Lloyd-Max only: the same for the 2 b1 plane
  float accf[NHB][8];      // folded float accumulators
  float ls[NHB];           // per-lane partial sum of p
  float carry[NHB][NG];    // rounding carry of this lane's P' digits, in [0, 1) units
  float zf[NHB][NG];       // float32 zero-point sum of the pages since the last flush into zacc
  int since_fold;          // pages since every head's accumulators were folded
};

// LDS of one history wave.  zacc holds each lane's partial sum of
// p * value zero in float64: the zero-point term is common to every channel
// of a group and large next to the output (it cancels against the code
// term), so the rounding of a long float32 chain would come back
// concentrated on a few channels after the rotation by R_V^T.  Pages add
// into a float32 register sum, flushed into zacc every 8 pages (a short
// chain); zacc lives in LDS to keep it out of the register budget.
template <int NHB, int NG>
struct HistSmem {
  int32_t pop[2][NHB * NG][kPage][4];   // P' digits: [page parity][head block x group][token][head]
  double zacc[NHB * NG][64];
  int32_t pt[64];                  // page-table entries pt_base .. pt_base + 63 of the split
};

// Fold the int32 accumulators of flagged heads into float, rescale to the
// new reference max and take a new P' unit from the current page.
// Float value, in units of the head's P' unit, of the accumulated P' .
// level products of channel block cb.
template <bool LM, int NHB, int G>
__device__ __forceinline__ float acc_value(const WaveState<NHB, G>& st, int hb, int cb, float ka, float kb) {
  // the j = 3 slots counted code - 2: add back 2 x their P' sums (both
  // code planes of the Lloyd-Max codebook carry the same offset)
  float corr = 0.f;
  if constexpr (WaveState<NHB, G>::kDcorr) corr = 2.f * p_digits(st.dcorr[hb][(16 * cb) / G]);
  if constexpr (LM) return ka * (p_digits(st.dacc[hb][cb]) + corr) + kb * (p_digits(st.dacc1[hb][cb]) + corr);
  else return p_digits(st.dacc[hb][cb]) + corr;
}

template <bool LM, int NHB, int G>
__device__ __forceinline__ void rebase(WaveState<NHB, G>& st, const float (&sc)[NHB][4],
                                    const uint32_t (&vsz)[4 * (kDim / G)], const bool (&need)[NHB],
                                    HistSmem<NHB, kDim / G>& sm, int lane, float ka, float kb) {
  constexpr int NG = kDim / G;
  // P' of this lane's tokens (residue j = n % 4 in the K-slot order) meets
  // codes masked in place, i.e. times 4^j (64 (code - 2) for j = 3): carry
  // 4^-j here
  const int jr = threadIdx.x & 3;
  const float slot = jr == 1 ? 0.25f : (jr == 2 ? 0.0625f : (jr == 3 ? 0.015625f : 1.f));
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float pm = row_reduce(fmaxf(fmaxf(sc[hb][0], sc[hb][1]), fmaxf(sc[hb][2], sc[hb][3])), MaxOp());
    const float m_new = need[hb] ? fmaxf(st.m_ref[hb], pm) : st.m_ref[hb];
    const float alpha = need[hb] ? exp2f(st.m_ref[hb] - m_new) : 1.f;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int gi = (16 * cb) / G;
      const float folded = (st.accf[hb][cb] + st.unit[hb][gi] * acc_value<LM>(st, hb, cb, ka, kb)) * alpha;
      st.accf[hb][cb] = need[hb] ? folded : st.accf[hb][cb];
      const v4i z = {0, 0, 0, 0};
      st.dacc[hb][cb] = need[hb] ? z : st.dacc[hb][cb];
      if constexpr (LM) st.dacc1[hb][cb] = need[hb] ? z : st.dacc1[hb][cb];
    }
    if constexpr (WaveState<NHB, G>::kDcorr) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const v4i z = {0, 0, 0, 0};
        st.dcorr[hb][gi] = need[hb] ? z : st.dcorr[hb][gi];
      }
    }
    st.ls[hb] *= alpha;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      sm.zacc[hb * NG + gi][lane] *= static_cast<double>(alpha);
      st.zf[hb][gi] *= alpha;
      float wmax = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float p = exp2f(sc[hb][m] - m_new);
        wmax = fmaxf(wmax, p * __uint_as_float(vsz[m * NG + gi] << 16));
      }
      wmax = row_reduce(wmax, MaxOp());
      const float u = fmaxf(wmax, 1e-30f) * (kHeadroom / kDigitUnitMax);
      st.unit[hb][gi] = need[hb] ? u : st.unit[hb][gi];
      st.carry[hb][gi] = need[hb] ? 0.5f : st.carry[hb][gi];
      st.inv[hb][gi] = need[hb] ? slot / u : st.inv[hb][gi];
    }
    st.m_ref[hb] = m_new;
  }
}

// Score half of a page: q . code, the online softmax and the P' digit rows
// of the page, written into P' slot `slot`.
template <bool LM, int NHB, int G>
__device__ __forceinline__ void score_page(WaveState<NHB, G>& st, const PageRegs<G>& cur, int tok_base,
                                           int n_hist, int lane, HistSmem<NHB, kDim / G>& sm, int slot,
                                           float lm_hi, float ka, float kb) {
  constexpr int NG = kDim / G;
  const int n = lane & 15, lg = lane >> 4;
  // ---- q . code: token tau(m, n) = 16 (n/4) + 4 m + n%4 in output column n;
  // sc holds scores / qs (the head's query unit is applied in the exponent)
  float sc[NHB][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const v4i b0 = unpack16(static_cast<uint32_t>(cur.kw[0][m]));
    const v4i b1 = unpack16(static_cast<uint32_t>(cur.kw[1][m]));
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float s;
      if constexpr (NG == 4) {
        // two groups per half: one product per group against the operand
        // masked to its channels (and, Lloyd-Max, the high-bit plane against
        // the masked second operand, as below)
        s = 0.f;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const v4i& bc = hf ? b1 : b0;
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qam[hb][hf][sub], bc, st.kc[hb][2 * hf + sub], 0, 0,
                                                          0);
            if constexpr (LM)
              d = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qbm[hb][hf][sub], high_bits(bc), d, 0, 0, 0);
            const int gi = 2 * hf + sub;
            const uint32_t sz = cur.ksz[m * NG + gi];
            const float ks = __uint_as_float(sz << 16);
            float kz = __uint_as_float(sz & 0xFFFF0000u);
            if constexpr (LM) kz = __builtin_fmaf(-lm_hi, ks, kz);
            s += __builtin_fmaf(ks, q_digits(d), kz * st.qz[hb][gi]);
          }
        }
      } else if constexpr (LM) {
        // level sum = ka * (q . c + (kb / ka) * q . 2 b1): the second operand
        // carries kb / ka, so both planes accumulate into one result, and qs
        // carries ka; zero - hi * scale takes the rest
        const v4i h0 = high_bits(b0), h1 = high_bits(b1);
        if constexpr (NG == 1) {
          v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][0], b0, st.kc[hb][0], 0, 0, 0);
          d = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][1], b1, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qb[hb][0], h0, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qb[hb][1], h1, d, 0, 0, 0);
          const uint32_t sz = cur.ksz[m];
          const float ks = __uint_as_float(sz << 16);
          const float kz = __builtin_fmaf(-lm_hi, ks, __uint_as_float(sz & 0xFFFF0000u));
          s = __builtin_fmaf(ks, q_digits(d), kz * st.qz[hb][0]);
        } else {
          v4i d0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][0], b0, st.kc[hb][0], 0, 0, 0);
          v4i d1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][1], b1, st.kc[hb][1], 0, 0, 0);
          d0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qb[hb][0], h0, d0, 0, 0, 0);
          d1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qb[hb][1], h1, d1, 0, 0, 0);
          const uint32_t s0 = cur.ksz[m * NG + 0], s1 = cur.ksz[m * NG + 1];
          const float ks0 = __uint_as_float(s0 << 16), ks1 = __uint_as_float(s1 << 16);
          const float kz0 = __builtin_fmaf(-lm_hi, ks0, __uint_as_float(s0 & 0xFFFF0000u));
          const float kz1 = __builtin_fmaf(-lm_hi, ks1, __uint_as_float(s1 & 0xFFFF0000u));
          s = __builtin_fmaf(ks0, q_digits(d0), kz0 * st.qz[hb][0]) +
              __builtin_fmaf(ks1, q_digits(d1), kz1 * st.qz[hb][1]);
        }
      } else if constexpr (NG == 1) {
        v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][0], b0, st.kc[hb][0], 0, 0, 0);
        d = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][1], b1, d, 0, 0, 0);
        const uint32_t sz = cur.ksz[m];
        s = __builtin_fmaf(__uint_as_float(sz << 16), q_digits(d),
                           __uint_as_float(sz & 0xFFFF0000u) * st.qz[hb][0]);
      } else {
        const v4i d0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][0], b0, st.kc[hb][0], 0, 0, 0);
        const v4i d1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][1], b1, st.kc[hb][1], 0, 0, 0);
        const uint32_t s0 = cur.ksz[m * NG + 0], s1 = cur.ksz[m * NG + 1];
        s = __builtin_fmaf(__uint_as_float(s0 << 16), q_digits(d0),
                           __uint_as_float(s0 & 0xFFFF0000u) * st.qz[hb][0]) +
            __builtin_fmaf(__uint_as_float(s1 << 16), q_digits(d1),
                           __uint_as_float(s1 & 0xFFFF0000u) * st.qz[hb][1]);
      }
      sc[hb][m] = s;
    }
  }
  // value scale/zero of this lane's tokens; on the request's last page the
  // slots past its end hold whatever the page held before (stale or never
  // written bytes, NaN or Inf included): their pairs are zeroed with their
  // scores, so a weight of 0 never meets them (0 * Inf and 0 * NaN are NaN)
  uint32_t vsz[4 * NG];
#pragma unroll
  for (int i = 0; i < 4 * NG; ++i) vsz[i] = cur.vsz[i];
  if (tok_base + kPage > n_hist) {   // the request's last page (uniform)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const bool valid = tok_base + 16 * (n >> 2) + 4 * m + (n & 3) < n_hist;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) sc[hb][m] = valid ? sc[hb][m] : -INFINITY;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) vsz[m * NG + gi] = valid ? vsz[m * NG + gi] : 0u;
    }
  }
  // ---- p against the reference max, P' in units of the head's fixed point
  float pr[NHB][4], xv[NHB][NG][4];
  float dmax = 0.f, xmax = 0.f;       // largest score above m, largest P' (this lane)
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    // (IEEE maximum: a score here is a finite product sum or the -inf of a
    // masked slot, so NaN handling does not matter, and unlike fmaxf it
    // needs no quieting of its operands)
    const float d = __builtin_fmaf(st.qs[hb],
                                   __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[hb][0], sc[hb][1]),
                                                                 __builtin_elementwise_maximum(sc[hb][2], sc[hb][3])),
                                   -st.m_ref[hb]);
    dmax = hb == 0 ? d : fmaxf(dmax, d);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      pr[hb][m] = __builtin_amdgcn_exp2f(__builtin_fmaf(st.qs[hb], sc[hb][m], -st.m_ref[hb]));   // 0 past the end
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        xv[hb][gi][m] = pr[hb][m] * __uint_as_float(vsz[m * NG + gi] << 16) * st.inv[hb][gi];
        xmax = fmaxf(xmax, xv[hb][gi][m]);
      }
    }
  }
  // ---- re-base the heads that need a new reference max or unit (rare),
  // and every head once its int32 accumulators have taken kFoldPages pages
  const uint64_t mask = __builtin_amdgcn_ballot_w64(dmax > kSlack) | __builtin_amdgcn_ballot_w64(xmax >= kDigitLimit);
  const bool force = ++st.since_fold >= kFoldPages;
  if (mask != 0 || force) {
    bool need[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) need[hb] = force || ((mask >> (16 * lg)) & 0xFFFFull) != 0;
    if (force) st.since_fold = 0;
    float sct[NHB][4];   // the scores themselves
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int m = 0; m < 4; ++m) sct[hb][m] = st.qs[hb] * sc[hb][m];
    rebase<LM, NHB, G>(st, sct, vsz, need, sm, lane, ka, kb);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        pr[hb][m] = __builtin_amdgcn_exp2f(sct[hb][m] - st.m_ref[hb]);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          xv[hb][gi][m] = pr[hb][m] * __uint_as_float(vsz[m * NG + gi] << 16) * st.inv[hb][gi];
      }
  }
  // ---- P' digits into the operand rows, l and zero-point partial sums
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int m = 0; m < 4; ++m) st.ls[hb] += pr[hb][m];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      uint32_t b[4];
      float zpage = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t sz = vsz[m * NG + gi];
        float vz = __uint_as_float(sz & 0xFFFF0000u);
        if constexpr (LM || !WaveState<NHB, G>::kDcorr) vz = __builtin_fmaf(st.zc, __uint_as_float(sz << 16), vz);
        zpage = __builtin_fmaf(pr[hb][m], vz, zpage);
        // floor with the carried fraction: the lane's rounded weights add up
        // to its exact ones within one unit
        const float t = xv[hb][gi][m] + st.carry[hb][gi];
        b[m] = static_cast<uint32_t>(t) + kDigitOffset;
        st.carry[hb][gi] = __builtin_amdgcn_fractf(t);
      }
      st.zf[hb][gi] += zpage;
      // a word per (token, head): the four digits of token tau(m, n) for
      // head lg; the value half reads them back transposed into rows
#pragma unroll
      for (int m = 0; m < 4; ++m)
        sm.pop[slot][hb * NG + gi][16 * (n >> 2) + 4 * m + (n & 3)][lg] = static_cast<int32_t>(b[m] ^ kLowDigitFlip);
    }
  }
  // every 8 pages the float32 zero-point sums go into the float64 ones
  if ((st.since_fold & 7) == 0) {   // uniform
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        sm.zacc[hb * NG + gi][lane] += static_cast<double>(st.zf[hb][gi]);
        st.zf[hb][gi] = 0.f;
      }
  }
}

// Value half of a page: P' . code of the page's value codes against the P'
// rows in slot `slot`, into the int32 accumulators.
template <bool LM, int NHB, int G>
__device__ __forceinline__ void value_page(WaveState<NHB, G>& st, const PageRegs<G>& cur, int lane,
                                           HistSmem<NHB, kDim / G>& sm, int slot) {
  constexpr int NG = kDim / G;
  const int n = lane & 15, lg = lane >> 4;
  // column n = channel 16 cb + n, rows = head x digit.  Lane (n, lg) needs
  // row n (head n/4, digit n%4) for the K slots of lane group lg: operand
  // byte e holds token 16 lg + 4 (e % 4) + e / 4.  Two transposed reads build
  // it from the [token][head] words: as a source, lane (n, lg) addresses the
  // words of heads 2 (n % 2), +1 for token 16 lg + 4 (i % 4) + i / 4 (i = n / 2),
  // then for that token + 2 (operand bytes 8..15).
  const int ti = n >> 1;
  const int t1 = 16 * lg + 4 * (ti & 3) + (ti >> 2), hp = 2 * (n & 1);
  v4i pa[NHB][NG];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const v2i lo = lds_read_tr8(&sm.pop[slot][hb * NG + gi][t1][hp]);
      const v2i hi = lds_read_tr8(&sm.pop[slot][hb * NG + gi][t1 + 2][hp]);
      pa[hb][gi] = v4i{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const int gi = (16 * cb) / G;
    const v4i bv = unpack16(static_cast<uint32_t>(cur.vw[cb >> 2][cb & 3]));
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      st.dacc[hb][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa[hb][gi], bv, st.dacc[hb][cb], 0, 0, 0);
    if constexpr (LM) {
      const v4i bh = high_bits(bv);
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        st.dacc1[hb][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa[hb][gi], bh, st.dacc1[hb][cb], 0, 0, 0);
    }
  }
  // the j = 3 P' digit sums of this page (64 x, every column alike)
  if constexpr (WaveState<NHB, G>::kDcorr) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
        st.dcorr[hb][gi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(pa[hb][gi], j3_ones(), st.dcorr[hb][gi], 0, 0, 0);
  }
}

// ---- bf16 sink/recent chunk on the matrix core ---------------------------
//
// One 64-slot chunk of the bf16 sink or recent tokens for query heads
// h_lo .. h_lo + nh - 1 (nh <= 4) of KV head kvh, request b, by one wave
// (page "超越TurboQuant：Together AI把2-bit KV Cache推向真实服务", section
// "OSCAR的另一个关键点是": sink and recent stay bf16 and meet the unrotated
// query).  The output is the chunk's normalised partial (natural-log LSE),
// the same as the vector-ALU chunk writes.
//   q . k on v_mfma_f32_16x16x32_bf16: rows = tokens (16 per block, four
//          blocks), columns = heads (four of 16 used), the K dimension =
//          channels; a lane's A operand is 16 contiguous bytes of one key
//          row, read straight from memory, and its B operand 16 bytes of
//          the query.  Products of bf16 values are exact in fp32.
//   p . v on the vector ALU: lane = (8-channel group, token residue mod 4),
//          16-byte loads along each value row, reduced over the residues.
// Every key load is issued at once (64 VGPRs), and the value rows two
// quarters ahead of their use, so the chunk waits on memory about twice
// instead of once per quarter row.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct Bf16MfmaSmem {
  float p[4][kPage];   // softmax numerators, [head][token]
};

__device__ __forceinline__ void bf16_chunk_mfma(const Bf16Params& a, int gq, int h_lo, int chunk, int kvh, int b,
                                                Bf16MfmaSmem& sm) {
  const int lane = threadIdx.x & 63, n = lane & 15, lg = lane >> 4;
  const int nh = min(4, gq - h_lo);
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
  const size_t kv0 = static_cast<size_t>(b) * a.hkv + kvh;
  const uint16_t* kb = chunk == 0 ? a.sink_k + kv0 * kSink * kDim
                                  : a.recent_k + (kv0 * kRecent + (chunk - 1) * kPage) * kDim;
  const uint16_t* vb = chunk == 0 ? a.sink_v + kv0 * kSink * kDim
                                  : a.recent_v + (kv0 * kRecent + (chunk - 1) * kPage) * kDim;
  // Loads through buffer resources that cover only the valid rows: a read
  // of a slot past n_valid (or of a head past nh) returns zeros, so those
  // slots need no address clamping, and stale bytes there (NaN or Inf
  // included) never reach the products.  Every offset goes in the
  // per-lane operand (with any constant part the compiler folds into the
  // instruction's offset field), which the range check covers; the scalar
  // offset operand is not checked and stays 0.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kb), 0, n_valid * kDim * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vb), 0, n_valid * kDim * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.q + head0 * kDim), 0, nh * kDim * 2, kRsrcWord3);
  // A operands: token 16 tb + n, channels 32 ks + 8 lg .. + 7; B operands:
  // head n, the same channels
  const uint32_t koff = static_cast<uint32_t>(n) * (kDim * 2) + static_cast<uint32_t>(lg) * 16u;
  v4i kr[4][4], qb[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kr[tb][ks] = load16r<false>(krs, koff + tb * 16 * kDim * 2 + ks * 64, 0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qb[ks] = load16r<false>(qrs, koff + ks * 64, 0);
  // d[tb][i] = q_n . k_t for token t = 16 tb + 4 lg + i
  v4f d[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    d[tb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      d[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kr[tb][ks]),
                                                      __builtin_bit_cast(v8bf, qb[ks]), d[tb], 0, 0, 0);
  }
  // value rows: quarter jq holds tokens res + 4 (4 jq + i), i = 0..3,
  // channels 8 cg .. 8 cg + 7; the first two quarters are requested before
  // the softmax, each later one while the quarter two before it is summed
  const int cg = lane & 15, res = lane >> 4;
  const uint32_t voff = static_cast<uint32_t>(res) * (kDim * 2) + static_cast<uint32_t>(cg) * 16u;
  auto load_quarter = [&](v4i (&vq)[4], int jq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vq[i] = load16r<false>(vrs, voff + (4 * jq + i) * 4 * kDim * 2, 0);
  };
  v4i va[4], vb4[4];
  load_quarter(va, 0);
  load_quarter(vb4, 1);
  // softmax per head over the 64 slots: head n's scores sit in lanes n,
  // n + 16, n + 32, n + 48 (16 each)
  float s[4][4];
  float mx = -INFINITY;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * lg + i;
      s[tb][i] = t < n_valid ? d[tb][i] * kScoreScaleLog2 : -INFINITY;
      mx = fmaxf(mx, s[tb][i]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));   // finite: slot 0 holds a token
  float ls = 0.f;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    float4 pv;
    pv.x = exp2f(s[tb][0] - mx);   // 0 for masked slots
    pv.y = exp2f(s[tb][1] - mx);
    pv.z = exp2f(s[tb][2] - mx);
    pv.w = exp2f(s[tb][3] - mx);
    ls += (pv.x + pv.y) + (pv.z + pv.w);
    if (n < 4) *reinterpret_cast<float4*>(&sm.p[n][16 * tb + 4 * lg]) = pv;
  }
  ls += __shfl_xor(ls, 16, 64);
  ls += __shfl_xor(ls, 32, 64);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float acc[4][8];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  auto sum_quarter = [&](const v4i (&vq)[4], int jq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = res + 4 * (4 * jq + i);
      const uint32_t ws[4] = {static_cast<uint32_t>(vq[i].x), static_cast<uint32_t>(vq[i].y),
                              static_cast<uint32_t>(vq[i].z), static_cast<uint32_t>(vq[i].w)};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float pt = sm.p[h][t];   // 0 past n_valid
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[h][2 * e] = __builtin_fmaf(pt, __uint_as_float(ws[e] << 16), acc[h][2 * e]);
          acc[h][2 * e + 1] = __builtin_fmaf(pt, __uint_as_float(ws[e] & 0xFFFF0000u), acc[h][2 * e + 1]);
        }
      }
    }
  };
  // (a loop, not unrolled: fully unrolled, the scheduler holds every value
  // word and numerator at once and exceeds the history kernel's budget)
#pragma unroll 1
  for (int jp = 0; jp < 2; ++jp) {   // uniform
    sum_quarter(va, 2 * jp);
    if (jp == 0) load_quarter(va, 2);
    sum_quarter(vb4, 2 * jp + 1);
    if (jp == 0) load_quarter(vb4, 3);
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    // head h's max and sum live in lane h
    const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), h));
    const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), h));
    const float inv = 1.f / lh;
    const size_t pidx = (head0 + h) * kBf16Parts + chunk;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (res == 0 && h < nh) a.po[pidx * kDim + cg * 8 + e] = v * inv;
    }
    if (lane == 0 && h < nh) a.plse[pidx] = (mh + log2f(lh)) * kLn2;
  }
}

// Issue priority of a wave by how far through its split's page groups it
// is: 3 in the first half, 2 to three quarters, 1 to seven eighths, 0 in
// the last eighth.  Waves sharing a SIMD otherwise issue oldest first, so of
// three equal splits started together the youngest finishes last and runs
// alone, with few loads in flight; a wave that gets ahead now yields to the
// ones behind it at each step, and the steps are closest together at the
// end, where the spread left over is what the launch waits for.
__device__ __forceinline__ void split_priority(int it, int groups) {   // uniform arguments
  if (2 * it < groups) __builtin_amdgcn_s_setprio(3);
  else if (4 * it < 3 * groups) __builtin_amdgcn_s_setprio(2);
  else if (8 * it < 7 * groups) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Orders one page's P' row writes before the reads that follow (a wave
// reads rows other lanes wrote).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One whole page, scores then values (slot 0).
template <bool LM, int NHB, int G>
__device__ __forceinline__ void process_page(WaveState<NHB, G>& st, const PageRegs<G>& cur, int tok_base,
                                             int n_hist, int lane, HistSmem<NHB, kDim / G>& sm,
                                             float lm_hi, float ka, float kb) {
  score_page<LM, NHB, G>(st, cur, tok_base, n_hist, lane, sm, 0, lm_hi, ka, kb);
  wave_lds_fence();
  value_page<LM, NHB, G>(st, cur, lane, sm, 0);
  wave_lds_fence();
}

template <int G, int WAVES, int BUF, int MINW, bool LM>
__global__ void __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(MINW)))
hist_mfma_kernel(MfmaParams a) {
  constexpr int NHB = 1;
  constexpr int NG = kDim / G;
  // non-temporal scale/zero loads pay only for the one-wave uniform G = 64
  // kernel (32 x 100K: 326.7 -> 320.9 us); at G = 128 (282.5 -> 287.9 us),
  // G = 32 (457 -> 471 us) and with the Lloyd-Max codebook they cost time
  constexpr bool kStreamSz = WAVES == 1 && G == 64 && !LM;
  // 1-D grid: every history split slot first (workgroups are dispatched in
  // id order, so these are the resident ones), then the bf16 chunks, which
  // fill the slots freed as history splits finish.  Slots beyond the
  // scheduled split count exit at once.  The chunks take only even ids
  // (the odd ones between them exit at once): workgroups go to the XCDs
  // round robin by id, and on the MI355X parts measured the even XCDs
  // finished their history splits 7-10 % sooner, so the chunks stay off the
  // slower ones.  A query group wider than four
  // heads takes two waves, heads 4w .. 4w+3 each; both read the same pages,
  // the second mostly from the compute unit's cache.
  const int id = blockIdx.x;
  const int n_hist_wg = a.slots * a.hkv;
  const int wave = WAVES == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
  const int lane = threadIdx.x & 63, n = lane & 15, lg = lane >> 4;
  union Smem {
    HistSmem<NHB, NG> hist[WAVES];
    Bf16MfmaSmem bf[WAVES];
  };
  __shared__ Smem smem;
  if (id >= n_hist_wg) {   // a bf16 sink/recent chunk, four heads per wave
    const int c0 = (n_hist_wg + 1) & ~1;   // first even id of the chunk range
    if (id < c0 || (id & 1)) return;
    const int r = (id - c0) >> 1;
    bf16_chunk_mfma(a.bf, a.gq, 4 * wave, r % kBf16Parts, (r / kBf16Parts) % a.hkv, r / (kBf16Parts * a.hkv),
                    smem.bf[wave]);
    return;
  }
  const int split = id / a.hkv, kvh = id % a.hkv;
  if (split >= a.sched[0]) return;
  // timing hook: shader-clock and constant-rate counters over workgroup 0
  const bool clk = a.clk != nullptr && id == 0;   // uniform
  unsigned long long clk0 = 0, wall0 = 0;
  if (clk) {
    clk0 = clock64();
    wall0 = wall_clock64();
  }
  // the split's request and page range, and the request's length, are
  // uniform: held in scalar registers so every branch on them is uniform
  const int b = __builtin_amdgcn_readfirstlane(a.sched[1 + 3 * split]);
  const int p0 = __builtin_amdgcn_readfirstlane(a.sched[2 + 3 * split]);
  const int p1 = __builtin_amdgcn_readfirstlane(a.sched[3 + 3 * split]);
  HistSmem<NHB, NG>& sm = smem.hist[wave];

  const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
  const int n_hist = max(0, L - kBf16Tokens);

  WaveState<NHB, G> st;
  const uint8_t* qp = a.qpack + (static_cast<size_t>(b) * a.hkv + kvh) * kQPackBytes;
  const float* qscale = reinterpret_cast<const float*>(qp + kQPackScaleOffset);
  const size_t head0 = static_cast<size_t>(b) * a.hq + static_cast<size_t>(kvh) * a.gq;
  bool head_ok[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const size_t off = ((hf * 4 + lg) * kQPackRows + (wave + hb) * 16 + n) * 16;
      st.qa[hb][hf] = *reinterpret_cast<const v4i*>(qp + off);
      if constexpr (LM) st.qb[hb][hf] = *reinterpret_cast<const v4i*>(qp + kQPackOperandBytes + off);
      if constexpr (NG == 4) {
        const v4i z = {0, 0, 0, 0};
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          st.qam[hb][hf][sub] = (lg >> 1) == sub ? st.qa[hb][hf] : z;
          if constexpr (LM) st.qbm[hb][hf][sub] = (lg >> 1) == sub ? st.qb[hb][hf] : z;
        }
      }
    }
    // q . code start values: 128 x the j = 3 digit sums of each product's
    // operands (two products against the +64 operand)
    {
      const v4i ones = j3_ones();
#pragma unroll
      for (int c = 0; c < NG; ++c) {
        v4i acc = {0, 0, 0, 0};
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
          if constexpr (NG == 1) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][hf], ones, acc, 0, 0, 0);
              if constexpr (LM) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qb[hb][hf], ones, acc, 0, 0, 0);
            }
          } else if constexpr (NG == 2) {
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qa[hb][c], ones, acc, 0, 0, 0);
            if constexpr (LM) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qb[hb][c], ones, acc, 0, 0, 0);
          } else {
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qam[hb][c >> 1][c & 1], ones, acc, 0, 0, 0);
            if constexpr (LM)
              acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.qbm[hb][c >> 1][c & 1], ones, acc, 0, 0, 0);
          }
        }
        st.kc[hb][c] = acc;
        if constexpr (WaveState<NHB, G>::kDcorr) st.dcorr[hb][c] = v4i{0, 0, 0, 0};
      }
    }
    const int h = 4 * (wave + hb) + lg;
    head_ok[hb] = h < a.gq;
    {
      // an all-zero query has unit 0 and zero sums: take 1, so scores / qs
      // stay 0 and a masked slot's -inf stays -inf
      const float u = LM ? qscale[h] * a.lm_ka : qscale[h];
      st.qs[hb] = u > 0.f ? u : 1.f;
    }
    st.m_ref[hb] = -INFINITY;
    st.ls[hb] = 0.f;
    st.since_fold = 0;
    // value zero of a token: zero - hi * scale (Lloyd-Max), and without the
    // extra products, + 2 (ka + kb or 1) * scale for the j = 3 tokens, whose
    // P' . code products counted code - 2
    {
      const bool j3 = (lane & 3) == 3;
      float zc = LM ? -a.lm_hi : 0.f;
      if constexpr (!WaveState<NHB, G>::kDcorr) zc += j3 ? 2.f * (LM ? a.lm_ka + a.lm_kb : 1.f) : 0.f;
      st.zc = zc;
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      st.qz[hb][gi] = head_ok[hb] ? a.qsum[(head0 + h) * 4 + gi] / st.qs[hb] : 0.f;
      st.unit[hb][gi] = 0.f;
      st.inv[hb][gi] = 0.f;
      sm.zacc[hb * NG + gi][lane] = 0.0;
      st.zf[hb][gi] = 0.f;
      st.carry[hb][gi] = 0.5f;
    }
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      st.dacc[hb][cb] = v4i{0, 0, 0, 0};
      if constexpr (LM) st.dacc1[hb][cb] = v4i{0, 0, 0, 0};
      st.accf[hb][cb] = 0.f;
    }
  }
  // Page-table entries of the split, 64 at a time in LDS (lane i writes
  // entry base + i), read back at a uniform address: the page addresses need
  // no dependent global load inside the loop, and the only wait on a global
  // load for them is at the refill every 64 pages.  (Holding them in a
  // register and broadcasting with readlane made the compiler wait for every
  // outstanding load before each page's address.)
  const int32_t* pt = a.page_table + static_cast<size_t>(b) * a.max_pages;
  const size_t blk_stride = static_cast<size_t>(a.hkv) * block_bytes(G);
  const uint8_t* base = a.pages + static_cast<size_t>(kvh) * block_bytes(G);
  int pt_base = p0;
  sm.pt[lane] = p0 + lane < p1 ? pt[p0 + lane] : 0;
  auto page_ptr = [&](int p) -> const uint8_t* {
    if (p - pt_base >= 64) {   // uniform: every lane sees the same p
      pt_base += 64;
      sm.pt[lane] = pt_base + lane < p1 ? pt[pt_base + lane] : 0;
    }
    const int phys = __builtin_amdgcn_readfirstlane(sm.pt[p - pt_base]);
    return base + static_cast<size_t>(phys) * blk_stride;
  };
  // BUF register page buffers: pages p+1 .. p+BUF-1 are in flight while p
  // is processed.  The inner loop is unrolled, so buffer indices are static.
  // Every step issues its loads (past the split's end it reloads the last
  // page, which the cache serves), so the count of loads between a page's
  // loads and its use is the same on every path and the compiler's wait
  // before a page can leave the younger pages in flight.  The loop leaves
  // only at its latch: an exit after any page would give the loop head a
  // path on which the youngest loads are the ones it needs first, and the
  // wait there would drain every page in flight.
  if (p0 < p1) {   // uniform
    const int p_last = p1 - 1;
    PageRegs<G> buf[BUF];
#pragma unroll
    for (int k = 0; k < BUF - 1; ++k) {
      load_page<G, WAVES == 1, kStreamSz>(buf[k], page_ptr(min(p0 + k, p_last)), lane);
      // keep the pages' loads in page order, the order the loop issues them
      // in: the loop head's wait then covers only the page it needs first
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (OSCAR_HIST_PIPE && G != 32) {
      // Software-pipelined: each step takes the value half of the previous
      // page (its matrix-core products) and then the score half of the next
      // one, so the products of one page can run while the vector work of the
      // next is issued.  P' rows alternate between two LDS slots by page
      // parity.  The first page has no value half before it; the last page's
      // value half follows the loop.  Page p0 + i lives in buf[i % BUF]; a
      // step's loads go into the buffer whose value half has just been taken.
      load_page<G, WAVES == 1, kStreamSz>(buf[BUF - 1], page_ptr(min(p0 + BUF - 1, p_last)), lane);
      score_page<LM, NHB, G>(st, buf[0], p0 * kPage, n_hist, lane, sm, 0, a.lm_hi, a.lm_ka, a.lm_kb);
      wave_lds_fence();
      // pages p0 + 1 .. in whole groups of BUF (one exit, at the latch)
      const int groups = (p1 - p0 - 1) / BUF;
      int p = p0 + 1;
      for (int it = 0; it < groups; ++it, p += BUF) {
        split_priority(it, groups);
#pragma unroll
        for (int k = 0; k < BUF; ++k) {
          value_page<LM, NHB, G>(st, buf[k % BUF], lane, sm, (p + k - 1 - p0) & 1);
          load_page<G, WAVES == 1, kStreamSz>(buf[k % BUF], page_ptr(min(p + k + BUF - 1, p_last)), lane);
          score_page<LM, NHB, G>(st, buf[(k + 1) % BUF], (p + k) * kPage, n_hist, lane, sm, (p + k - p0) & 1, a.lm_hi,
                                 a.lm_ka, a.lm_kb);
          wave_lds_fence();
        }
      }
      // the remaining (p1 - p0 - 1) % BUF pages are already loaded
      const int rem = (p1 - p0 - 1) % BUF;
#pragma unroll
      for (int k = 0; k < BUF - 1; ++k)
        if (k < rem) {
          value_page<LM, NHB, G>(st, buf[k % BUF], lane, sm, (p + k - 1 - p0) & 1);
          score_page<LM, NHB, G>(st, buf[(k + 1) % BUF], (p + k) * kPage, n_hist, lane, sm, (p + k - p0) & 1, a.lm_hi,
                                 a.lm_ka, a.lm_kb);
          wave_lds_fence();
        }
      // the last page's value half: page p1 - 1 = p0 + groups * BUF + rem, in buf[rem]
#pragma unroll
      for (int k = 0; k < BUF; ++k)
        if (k == rem) value_page<LM, NHB, G>(st, buf[k], lane, sm, (p1 - 1 - p0) & 1);
      wave_lds_fence();
    } else {
      // whole groups of BUF pages: one exit, at the latch, so the loads in
      // flight at the loop head are the same on every path into it
      const int groups = (p1 - p0) / BUF;
      int p = p0;
      for (int it = 0; it < groups; ++it, p += BUF) {
        split_priority(it, groups);
#pragma unroll
        for (int k = 0; k < BUF; ++k) {
          load_page<G, WAVES == 1, kStreamSz>(buf[(k + BUF - 1) % BUF], page_ptr(min(p + k + BUF - 1, p_last)), lane);
          process_page<LM, NHB, G>(st, buf[k], (p + k) * kPage, n_hist, lane, sm, a.lm_hi, a.lm_ka, a.lm_kb);
        }
      }
      // the last (p1 - p0) % BUF pages are already in buf[0 ..]
#pragma unroll
      for (int k = 0; k < BUF - 1; ++k)
        if (p + k < p1)
          process_page<LM, NHB, G>(st, buf[k], (p + k) * kPage, n_hist, lane, sm, a.lm_hi, a.lm_ka, a.lm_kb);
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // ---- partial output of this split (rotated value domain)
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float l = row_reduce(st.ls[hb], AddOp());
    double zsum[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      zsum[gi] = row_sum_f64(sm.zacc[hb * NG + gi][lane] + static_cast<double>(st.zf[hb][gi]));
    }
    if (!head_ok[hb]) continue;
    const int h = 4 * (wave + hb) + lg;
    const size_t pidx = static_cast<size_t>(split) * a.hq + static_cast<size_t>(kvh) * a.gq + h;
    const bool any = l > 0.f;
    const float inv_l = any ? 1.f / l : 0.f;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int gi = (16 * cb) / G;
      const double o =
          static_cast<double>(st.accf[hb][cb] + st.unit[hb][gi] * acc_value<LM>(st, hb, cb, a.lm_ka, a.lm_kb)) +
          zsum[gi];
      a.po[pidx * kDim + 16 * cb + n] = static_cast<float>(o) * inv_l;
    }
    if (n == 0) a.plse[pidx] = any ? (st.m_ref[hb] + log2f(l)) * kLn2 : -INFINITY;
  }
  if (clk && threadIdx.x == 0) {
    const unsigned long long clk1 = clock64(), wall1 = wall_clock64();
    a.clk[0] = clk0;
    a.clk[1] = wall0;
    a.clk[2] = clk1;
    a.clk[3] = wall1;
  }
}

// Register page buffers and waves per SIMD of each instantiation: the
// G = 128 uniform kernels run three waves per SIMD with two buffers; the
// other uniform kernels keep two buffers at two waves per SIMD (a third
// buffer measured 1-2 % slower, and G = 64 fits a third wave only with one
// buffer, 3 % slower); the Lloyd-Max kernels keep two buffers (one at
// G = 32, where two spill) at two waves.
template <int G, int WAVES, bool LM>
struct HistShape {
  // G = 128 uniform kernels fit three waves per SIMD (168 VGPRs, no spills):
  // GQA-8 about 7 % faster than at two; GQA <= 4 about 0.6 % (32 x 100K:
  // 279.8-280.9 against 281.7-282.4 us, same box)
  static constexpr bool kThreeWaves = G == 128 && !LM;
  static constexpr int BUF = G == 32 ? (LM ? 1 : OSCAR_HIST_BUFFERS_32) : kThreeWaves ? 2
                                     : (LM ? OSCAR_HIST_BUFFERS_LM : OSCAR_HIST_BUFFERS);
  static constexpr int MINW = kThreeWaves ? 3 : (LM ? OSCAR_HIST_MIN_WAVES_LM : OSCAR_HIST_MIN_WAVES);
};

template <int G, int WAVES, bool LM>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  constexpr int BUF = HistShape<G, WAVES, LM>::BUF;
  constexpr int MINW = HistShape<G, WAVES, LM>::MINW;
  const oscar_dims& d = *a.dims;
  MfmaParams p;
  p.pages = a.cache->pages;
  p.page_table = a.cache->page_table;
  p.seq_lens = a.cache->seq_lens;
  p.qpack = a.ws + a.lay.off_qpack;
  p.qsum = reinterpret_cast<const float*>(a.ws + a.lay.off_qsum);
  p.sched = reinterpret_cast<const int32_t*>(a.ws + a.lay.off_sched);
  p.po = reinterpret_cast<float*>(a.ws + a.lay.off_ho);
  p.plse = reinterpret_cast<float*>(a.ws + a.lay.off_hlse);
  p.max_pages = a.cache->max_pages_per_req;
  p.hkv = d.num_kv_heads;
  p.hq = d.num_q_heads;
  p.gq = d.num_q_heads / d.num_kv_heads;
  p.slots = a.hist_slots > 0 ? a.hist_slots : a.lay.slots;
  const Codebook* cbk = codebook_of(d.codebook);
  p.lm_hi = cbk->lev[3];
  p.lm_ka = cbk->lev[3] - cbk->lev[2];
  p.lm_kb = (3.f * cbk->lev[2] - cbk->lev[3]) * 0.5f;
  p.bf = make_bf16_params(a);
  p.clk = a.clock_trace;
  const int n_hist_wg = p.slots * d.num_kv_heads;
  const dim3 grid(((n_hist_wg + 1) & ~1) + 2 * kBf16Parts * a.cache->batch * d.num_kv_heads);
  const dim3 block(64 * WAVES);
  if (a.ev_start != nullptr && a.ev_stop != nullptr)
    hipExtLaunchKernelGGL(hist_mfma_kernel<G, WAVES, BUF, MINW, LM>, grid, block, 0, s, a.ev_start, a.ev_stop, 0,
                          p);
  else
    hist_mfma_kernel<G, WAVES, BUF, MINW, LM><<<grid, block, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

int hist_default_target(const oscar_dims& d, int simds) {
  // the workgroups the matrix-core kernel for these dims keeps resident:
  // SIMDs x waves per SIMD / waves per workgroup
  const bool two = d.num_q_heads / d.num_kv_heads > 4;
  const bool lm = d.codebook == OSCAR_CODEBOOK_LLOYD_MAX;
  int waves;
  if (d.group_size == 128) {
    if (lm) waves = two ? HistShape<128, 2, true>::MINW : HistShape<128, 1, true>::MINW;
    else waves = two ? HistShape<128, 2, false>::MINW : HistShape<128, 1, false>::MINW;
  } else if (d.group_size == 32) {
    if (lm) waves = two ? HistShape<32, 2, true>::MINW : HistShape<32, 1, true>::MINW;
    else waves = two ? HistShape<32, 2, false>::MINW : HistShape<32, 1, false>::MINW;
  } else {
    if (lm) waves = two ? HistShape<64, 2, true>::MINW : HistShape<64, 1, true>::MINW;
    else waves = two ? HistShape<64, 2, false>::MINW : HistShape<64, 1, false>::MINW;
  }
  return simds * waves / (two ? 2 : 1);
}

bool hist_mfma_supported(const oscar_dims& d) {
  const int g = d.num_q_heads / d.num_kv_heads;
  return (d.group_size == 32 || d.group_size == 64 || d.group_size == 128) && g >= 1 && g <= 8;
}

hipError_t launch_hist_mfma(const DecodeArgs& a, hipStream_t s) {
  const int g = a.dims->num_q_heads / a.dims->num_kv_heads;
  const bool two = g > 4;
  if (a.dims->codebook == OSCAR_CODEBOOK_LLOYD_MAX) {
    if (a.dims->group_size == 32) return two ? launch_t<32, 2, true>(a, s) : launch_t<32, 1, true>(a, s);
    if (a.dims->group_size == 64) return two ? launch_t<64, 2, true>(a, s) : launch_t<64, 1, true>(a, s);
    return two ? launch_t<128, 2, true>(a, s) : launch_t<128, 1, true>(a, s);
  }
  if (a.dims->group_size == 32) return two ? launch_t<32, 2, false>(a, s) : launch_t<32, 1, false>(a, s);
  if (a.dims->group_size == 64) return two ? launch_t<64, 2, false>(a, s) : launch_t<64, 1, false>(a, s);
  return two ? launch_t<128, 2, false>(a, s) : launch_t<128, 1, false>(a, s);
}

}  // namespace oscar
