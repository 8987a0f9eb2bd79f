// Plain C++ CPU oracle of OSCAR's INT2 KV-cache decode path, float64.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
// baseline of the benchmark load this library.  It shares no code, header,
// table or constant with the HIP library and includes nothing from it.
//
// What it computes, per (request, KV head): demote every history token
// (rotate by R in float64 rounded once to float32, clip per channel, quantize
// each group of G channels to one of four levels with bfloat16 scale and zero
// point), dequantize, and attend once over sink + history + recent in
// float64.  Each step is written the direct way: one token at a time, one sum
// in index order, no blocking and no reordering.  The one liberty is that a
// history token is dequantized where it is used instead of being kept: the
// keys in a first pass (scores), the values in a second pass (weighted sum),
// which changes no value.  The only parallelism is an OpenMP loop over
// independent (request, KV head) pairs.
//
// Sources (short labels as in the numpy oracle):
//   [A] "Together AI 开源 OSCAR：一种面向长上下文 LLM 服务的注意力感知 2 位 KV
//       缓存量化系统" (news.chathome.org)
//   [B] "超越TurboQuant：Together AI把2-bit KV Cache推向真实服务" (haoling.cc)
//   [C] "OSCAR: открытая система двухбитного сжатия KV-кэша" (Telegram post)
//
// Readings where the pages are silent are the numpy oracle's, restated at
// each function.  Parity status: pinned by CPU tests against the numpy
// oracle (codes, scales and zero points bit-exact, outputs to 1e-12),
// against brute-force attention when there is no history, and against the
// four-level Gaussian Lloyd-Max quantizer's published levels.
//
// Errors: every entry point returns 0 on success and -22 (EINVAL) for a
// null pointer, a group other than 32, 64 or 128, a codebook other than 0
// (uniform) or 1 (Lloyd-Max), or a negative count.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include <omp.h>

namespace {

constexpr int kDim = 128;     // head dimension of every model the pages evaluate
constexpr int kSink = 64;     // bf16 sink tokens: [A] §服务系统：混合精度缓存布局; [B]; [C]
constexpr int kRecent = 256;  // bf16 recent window, same places
constexpr int kLevels = 4;    // INT2: [A] §为什么 INT2 KV 缓存量化很难？
constexpr int kEinval = -22;

// ---------------------------------------------------------------------------
// bfloat16

double bf16_to_double(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return double(f);
}

// Nearest bfloat16 (ties to even) of a float32, returned as a float32.
float bf16_round(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  uint64_t w = u;
  uint64_t lsb = (w >> 16) & 1u;
  uint32_t r = uint32_t(((w + 0x7FFFu + lsb) >> 16) << 16);
  float f;
  std::memcpy(&f, &r, 4);
  return f;
}

// ---------------------------------------------------------------------------
// Lloyd-Max quantizer of N(0, 1) ([B], the paragraph comparing OSCAR with
// TurboQuant, says OSCAR's code pairs its rotation with a Lloyd-Max codebook).
// READING: the four-level minimum-MSE quantizer of the standard normal.
// Lloyd's alternation on the positive half (the optimum is symmetric):
// thresholds at the midpoints of adjacent levels, each level the mean of the
// normal restricted to its cell, (pdf(a) - pdf(b)) / P(a < X < b).  Start at
// 1/2, 3/2; stop once no level moves by more than 1e-15, after one more pass.

double normal_pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

double normal_tail(double x) {  // P(X > x)
  return std::isinf(x) ? 0.0 : 0.5 * std::erfc(x / std::sqrt(2.0));
}

void lloyd_max(double levels[kLevels], double thresholds[kLevels - 1]) {
  constexpr int half = kLevels / 2;
  double lev[half];
  for (int k = 0; k < half; ++k) lev[k] = k + 0.5;
  int extra = 1;
  for (int it = 0; it < 100000; ++it) {
    double edge[half + 1];
    edge[0] = 0.0;
    for (int k = 1; k < half; ++k) edge[k] = 0.5 * (lev[k - 1] + lev[k]);
    edge[half] = INFINITY;
    double moved = 0.0;
    double next[half];
    for (int k = 0; k < half; ++k) {
      double a = edge[k], b = edge[k + 1];
      double pb = std::isinf(b) ? 0.0 : normal_pdf(b);
      next[k] = (normal_pdf(a) - pb) / (normal_tail(a) - normal_tail(b));
      moved = std::fmax(moved, std::fabs(next[k] - lev[k]));
    }
    for (int k = 0; k < half; ++k) lev[k] = next[k];
    if (moved <= 1e-15) {
      if (extra == 0) break;
      --extra;
    }
  }
  for (int k = 0; k < half; ++k) {
    levels[half + k] = lev[k];
    levels[half - 1 - k] = -lev[k];
  }
  for (int k = 0; k + 1 < kLevels; ++k) thresholds[k] = 0.5 * (levels[k] + levels[k + 1]);
}

struct Codebook {
  float level[kLevels];      // stored levels, float32
  float thresh[kLevels - 1]; // decision thresholds, float32
};

Codebook make_codebook() {
  double lev[kLevels], thr[kLevels - 1];
  lloyd_max(lev, thr);
  Codebook cb;
  for (int k = 0; k < kLevels; ++k) cb.level[k] = float(lev[k]);
  for (int k = 0; k + 1 < kLevels; ++k) cb.thresh[k] = float(thr[k]);
  return cb;
}

// ---------------------------------------------------------------------------
// Demotion of one token ([B] §OSCAR的另一个关键点是: rotate, clip, quantize).

// y = x . R: the bf16 token times the float32 rotation, summed in float64 in
// index order and rounded once to float32; then clamped to [-c_k, c_k].
void rotate_clip(const uint16_t* x_bits, const float* r, const float* clip, float y[kDim]) {
  double x[kDim];
  for (int i = 0; i < kDim; ++i) x[i] = bf16_to_double(x_bits[i]);
  for (int k = 0; k < kDim; ++k) {
    double acc = 0.0;
    for (int i = 0; i < kDim; ++i) acc += x[i] * double(r[i * kDim + k]);
    float v = float(acc);
    float c = clip[k];
    y[k] = std::fmin(std::fmax(v, -c), c);
  }
}

// Uniform asymmetric INT2 per group ([A] §为什么 INT2 KV 缓存量化很难？ four
// levels; [B] §OSCAR的另一个关键点是 scale and zero point).  READING: zero =
// group minimum, scale = (max - min) / 3, both rounded to bfloat16; code =
// clamp(rint((y - zero) / scale), 0, 3) in float32 with ties to even; a group
// whose scale is 0 gets code 0.
void quantize_uniform(const float* y, int group, uint8_t* code, float* scale, float* zero) {
  float mn = y[0], mx = y[0];
  for (int i = 1; i < group; ++i) {
    mn = std::fmin(mn, y[i]);
    mx = std::fmax(mx, y[i]);
  }
  float range = mx - mn;
  float s = bf16_round(range / 3.0f);
  float z = bf16_round(mn);
  for (int i = 0; i < group; ++i) {
    if (s == 0.0f) {
      code[i] = 0;
      continue;
    }
    float diff = y[i] - z;
    float t = diff / s;
    double c = std::nearbyint(double(t));
    if (c < 0) c = 0;
    if (c > kLevels - 1) c = kLevels - 1;
    code[i] = uint8_t(c);
  }
  *scale = s;
  *zero = z;
}

// Lloyd-Max per group.  READING: zero = group mean, scale = population
// standard deviation (both float64, rounded to float32, then to bfloat16);
// u = (y - zero) / scale in float32; the code is the number of float32
// thresholds strictly below u; scale 0 gives code 0.
void quantize_lloyd(const float* y, int group, const Codebook& cb, uint8_t* code, float* scale,
                    float* zero) {
  double sum = 0.0;
  for (int i = 0; i < group; ++i) sum += double(y[i]);
  double mean = sum / group;
  double sq = 0.0;
  for (int i = 0; i < group; ++i) sq += (double(y[i]) - mean) * (double(y[i]) - mean);
  double var = sq / group;
  float z = bf16_round(float(mean));
  float s = bf16_round(float(std::sqrt(var)));
  for (int i = 0; i < group; ++i) {
    if (s == 0.0f) {
      code[i] = 0;
      continue;
    }
    float diff = y[i] - z;
    float u = diff / s;
    int c = 0;
    for (int k = 0; k + 1 < kLevels; ++k) c += (u > cb.thresh[k]) ? 1 : 0;
    code[i] = uint8_t(c);
  }
  *scale = s;
  *zero = z;
}

void demote_token(const uint16_t* x_bits, const float* r, const float* clip, int group, int codebook,
                  const Codebook& cb, uint8_t code[kDim], float* scale, float* zero) {
  float y[kDim];
  rotate_clip(x_bits, r, clip, y);
  for (int g0 = 0, gi = 0; g0 < kDim; g0 += group, ++gi) {
    if (codebook == 0)
      quantize_uniform(y + g0, group, code + g0, scale + gi, zero + gi);
    else
      quantize_lloyd(y + g0, group, cb, code + g0, scale + gi, zero + gi);
  }
}

// Dequantized stored-domain value of one token: code * scale + zero in
// float32 (uniform; code * scale is exact), zero + scale * level[code] in
// float64 (Lloyd-Max).
void dequantize_token(const uint8_t code[kDim], const float* scale, const float* zero, int group,
                      int codebook, const Codebook& cb, double out[kDim]) {
  for (int i = 0; i < kDim; ++i) {
    int gi = i / group;
    if (codebook == 0)
      out[i] = double(float(code[i]) * scale[gi] + zero[gi]);
    else
      out[i] = double(zero[gi]) + double(scale[gi]) * double(cb.level[code[i]]);
  }
}

bool valid_group(int group) { return group == 32 || group == 64 || group == 128; }

}  // namespace

extern "C" {

// One (request, KV head) pair for the batched entry point.
struct OscarOraclePair {
  const uint16_t* q;        // [g][128] bf16 bits, the g query heads of this KV head
  const uint16_t* k;        // token t's key at k + t * token_stride (bf16 bits)
  const uint16_t* v;        // same for values
  int64_t len;              // L, tokens held by the request (the appended one included)
  int64_t token_stride;     // elements between successive tokens
  const float* r_k;         // [128][128] float32, row-major: y = x . R
  const float* r_v;
  const float* clip_k;      // [128] float32
  const float* clip_v;
  double* out;              // [g][128]
  double* lse;              // [g], natural log
};

// The Lloyd-Max levels [4] and thresholds [3] of N(0, 1), float64.
int oscar_oracle_lloyd_max(double* levels, double* thresholds) {
  if (!levels || !thresholds) return kEinval;
  lloyd_max(levels, thresholds);
  return 0;
}

// Demote n tokens of one KV head: x_bits [n][128] bf16 bits; r [128][128];
// clip [128]; codes out [n][128] (0..3), scale and zero out [n][128/group]
// float32 (bfloat16 values).
int oscar_oracle_demote(const uint16_t* x_bits, int64_t n, const float* r, const float* clip,
                        int32_t group, int32_t codebook, uint8_t* codes, float* scale, float* zero) {
  if (n < 0 || !valid_group(group) || (codebook != 0 && codebook != 1)) return kEinval;
  if (n > 0 && (!x_bits || !r || !clip || !codes || !scale || !zero)) return kEinval;
  const Codebook cb = make_codebook();
  const int ng = kDim / group;
  for (int64_t t = 0; t < n; ++t)
    demote_token(x_bits + t * kDim, r, clip, group, codebook, cb, codes + t * kDim, scale + t * ng,
                 zero + t * ng);
  return 0;
}

}  // extern "C"

namespace {

// Attention of the g query heads of one KV head after the request's latest
// append and demotion.  Regions: the first 64 tokens and the last 256
// (after the first 64) stay bf16; tokens 64 .. L-257 are history, demoted
// one by one.  Keys are stored as K R_K, so a history score is (q R_K) . k_hat;
// values are stored as V R_V, so the history part of the output is
// (sum_t p_t v_hat_t) R_V^T.  One softmax over all tokens with scale
// 1/sqrt(128) ([B] §OSCAR的另一个关键点是; [A] §服务系统：混合精度缓存布局).
void request_head(const OscarOraclePair& pr, int g, int group, int codebook, const Codebook& cb) {
  const int64_t L = pr.len;
  const int64_t n_sink = L < kSink ? L : kSink;
  const int64_t n_hist = L - (kSink + kRecent) > 0 ? L - (kSink + kRecent) : 0;
  int64_t n_recent = L - kSink > 0 ? L - kSink : 0;
  if (n_recent > kRecent) n_recent = kRecent;
  const int ng = kDim / group;
  const double inv_sqrt_d = 1.0 / std::sqrt(double(kDim));

  // bf16 positions: the sink, then the recent window.
  std::vector<int64_t> bpos;
  for (int64_t t = 0; t < n_sink; ++t) bpos.push_back(t);
  for (int64_t t = L - n_recent; t < L; ++t) bpos.push_back(t);
  const int64_t nb = int64_t(bpos.size());

  std::vector<double> q(size_t(g) * kDim), qr(size_t(g) * kDim);
  for (int h = 0; h < g; ++h) {
    for (int i = 0; i < kDim; ++i) q[h * kDim + i] = bf16_to_double(pr.q[h * kDim + i]);
    for (int k = 0; k < kDim; ++k) {
      double acc = 0.0;
      for (int i = 0; i < kDim; ++i) acc += q[h * kDim + i] * double(pr.r_k[i * kDim + k]);
      qr[h * kDim + k] = acc;
    }
  }

  // Pass 1: every score.
  std::vector<double> sb(size_t(g) * nb), sh(size_t(g) * n_hist);
  for (int64_t j = 0; j < nb; ++j) {
    const uint16_t* kt = pr.k + bpos[j] * pr.token_stride;
    for (int h = 0; h < g; ++h) {
      double acc = 0.0;
      for (int i = 0; i < kDim; ++i) acc += q[h * kDim + i] * bf16_to_double(kt[i]);
      sb[h * nb + j] = acc * inv_sqrt_d;
    }
  }
  uint8_t code[kDim];
  std::vector<float> sc(ng), zp(ng);
  double deq[kDim];
  for (int64_t j = 0; j < n_hist; ++j) {
    demote_token(pr.k + (kSink + j) * pr.token_stride, pr.r_k, pr.clip_k, group, codebook, cb, code,
                 sc.data(), zp.data());
    dequantize_token(code, sc.data(), zp.data(), group, codebook, cb, deq);
    for (int h = 0; h < g; ++h) {
      double acc = 0.0;
      for (int i = 0; i < kDim; ++i) acc += qr[h * kDim + i] * deq[i];
      sh[h * n_hist + j] = acc * inv_sqrt_d;
    }
  }

  // Pass 2: softmax weights and the weighted value sums.
  std::vector<double> m(g, -INFINITY), denom(g, 0.0);
  for (int h = 0; h < g; ++h) {
    for (int64_t j = 0; j < nb; ++j) m[h] = std::fmax(m[h], sb[h * nb + j]);
    for (int64_t j = 0; j < n_hist; ++j) m[h] = std::fmax(m[h], sh[h * n_hist + j]);
  }
  std::vector<double> ob(size_t(g) * kDim, 0.0), oh(size_t(g) * kDim, 0.0);
  for (int64_t j = 0; j < nb; ++j) {
    const uint16_t* vt = pr.v + bpos[j] * pr.token_stride;
    for (int h = 0; h < g; ++h) {
      double p = std::exp(sb[h * nb + j] - m[h]);
      denom[h] += p;
      for (int i = 0; i < kDim; ++i) ob[h * kDim + i] += p * bf16_to_double(vt[i]);
    }
  }
  for (int64_t j = 0; j < n_hist; ++j) {
    demote_token(pr.v + (kSink + j) * pr.token_stride, pr.r_v, pr.clip_v, group, codebook, cb, code,
                 sc.data(), zp.data());
    dequantize_token(code, sc.data(), zp.data(), group, codebook, cb, deq);
    for (int h = 0; h < g; ++h) {
      double p = std::exp(sh[h * n_hist + j] - m[h]);
      denom[h] += p;
      for (int i = 0; i < kDim; ++i) oh[h * kDim + i] += p * deq[i];
    }
  }
  // Un-rotate the history part: (oh R_V^T)_c = sum_k oh_k R_V[c][k].
  for (int h = 0; h < g; ++h) {
    for (int c = 0; c < kDim; ++c) {
      double acc = 0.0;
      for (int k = 0; k < kDim; ++k) acc += oh[h * kDim + k] * double(pr.r_v[c * kDim + k]);
      pr.out[h * kDim + c] = (ob[h * kDim + c] + acc) / denom[h];
    }
    pr.lse[h] = m[h] + std::log(denom[h]);
  }
}

}  // namespace

extern "C" {

// Attention output of n_pairs independent (request, KV head) pairs, each
// with g query heads, on `threads` OpenMP threads (pairs handed out one at a
// time).  Every pair needs len >= 1 (a decode step has appended a token).
int oscar_oracle_attend_pairs(const OscarOraclePair* pairs, int32_t n_pairs, int32_t g,
                              int32_t group, int32_t codebook, int32_t threads) {
  if (n_pairs < 0 || g < 1 || threads < 1 || !valid_group(group) || (codebook != 0 && codebook != 1))
    return kEinval;
  if (n_pairs > 0 && !pairs) return kEinval;
  for (int32_t i = 0; i < n_pairs; ++i) {
    const OscarOraclePair& p = pairs[i];
    if (p.len < 1 || p.token_stride < kDim || !p.q || !p.k || !p.v || !p.r_k || !p.r_v ||
        !p.clip_k || !p.clip_v || !p.out || !p.lse)
      return kEinval;
  }
  const Codebook cb = make_codebook();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
  for (int32_t i = 0; i < n_pairs; ++i) request_head(pairs[i], g, group, codebook, cb);
  return 0;
}

}  // extern "C"
