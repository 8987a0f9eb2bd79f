// Codebooks of the 2-bit history codes (host side).
//
// The Lloyd-Max codebook is the 4-level minimum-mean-squared-error quantizer
// of the standard normal distribution.  Its two conditions (each level is
// the mean of the distribution over its cell; each decision threshold is
// the midpoint of its two levels) reduce, by symmetry, to one equation in
// the positive threshold t:
//   t = (lo(t) + hi(t)) / 2,   lo(t) = E[X | 0 < X < t],  hi(t) = E[X | X > t],
// with E[X | a < X < b] = (pdf(a) - pdf(b)) / P(a < X < b) for X ~ N(0, 1).
// g(t) = (lo(t) + hi(t)) / 2 - t is positive at t = 1/2 and negative at
// t = 3/2; bisection on that bracket finds the root to float64 resolution.
// The stored codebook is the float32 rounding of the levels and of the
// midpoints of adjacent float64 levels.
#include <math.h>

#include "oscar_internal.h"

namespace oscar {
namespace {

double normal_pdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }
double normal_upper_tail(double x) { return 0.5 * erfc(x / sqrt(2.0)); }

double cell_mean_low(double t) { return (normal_pdf(0.0) - normal_pdf(t)) / (0.5 - normal_upper_tail(t)); }
double cell_mean_high(double t) { return normal_pdf(t) / normal_upper_tail(t); }

Codebook make_lloyd_max() {
  double a = 0.5, b = 1.5;   // g(a) > 0 > g(b)
  for (int it = 0; it < 200; ++it) {
    const double m = 0.5 * (a + b);
    if (m <= a || m >= b) break;
    const double g = 0.5 * (cell_mean_low(m) + cell_mean_high(m)) - m;
    if (g > 0.0) a = m;
    else b = m;
  }
  const double t = 0.5 * (a + b);
  const double lo = cell_mean_low(t), hi = cell_mean_high(t);
  Codebook c;
  c.lev[0] = static_cast<float>(-hi);
  c.lev[1] = static_cast<float>(-lo);
  c.lev[2] = static_cast<float>(lo);
  c.lev[3] = static_cast<float>(hi);
  const double mid = 0.5 * (lo + hi);
  c.thr[0] = static_cast<float>(-mid);
  c.thr[1] = 0.0f;
  c.thr[2] = static_cast<float>(mid);
  return c;
}

}  // namespace

const Codebook* codebook_of(int32_t codebook) {
  static const Codebook uniform = {{0.f, 1.f, 2.f, 3.f}, {0.5f, 1.5f, 2.5f}};
  static const Codebook lloyd = make_lloyd_max();
  if (codebook == OSCAR_CODEBOOK_UNIFORM) return &uniform;
  if (codebook == OSCAR_CODEBOOK_LLOYD_MAX) return &lloyd;
  return nullptr;
}

}  // namespace oscar

extern "C" int oscar_codebook(int32_t codebook, float* levels, float* thresholds) {
  const oscar::Codebook* c = oscar::codebook_of(codebook);
  if (c == nullptr) return OSCAR_EUNSUPPORTED;
  for (int i = 0; i < 4 && levels != nullptr; ++i) levels[i] = c->lev[i];
  for (int i = 0; i < 3 && thresholds != nullptr; ++i) thresholds[i] = c->thr[i];
  return OSCAR_OK;
}
