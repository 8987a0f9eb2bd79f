// Offline calibration of the OSCAR rotations and clip thresholds
// (page "Together AI 开源 OSCAR：一种面向长上下文 LLM 服务的注意力感知 2 位 KV
// 缓存量化系统", section "OSCAR 的不同之处"; page "超越TurboQuant：Together AI把
// 2-bit KV Cache推向真实服务", section "OSCAR把旋转对准attention"):
//   C_Q = mean of q^T q over the calibration queries of a KV head's group,
//   C_S = mean of o^T o with o = S V the causal attention outputs (so that
//         C_S = V^T S^T S V / N),
//   R   = U . H . P_br with U the eigenvectors of C (eigenvalues descending),
//         H the normalised Sylvester Hadamard matrix and P_br the 7-bit
//         bit-reversal permutation,
//   clip = per-channel percentile of |x . R| over the calibration tokens.
// The O(N^2 d) and O(N d^2) statistics run in float64 HIP kernels; the
// 128x128 symmetric eigenproblems are solved on the host by cyclic Jacobi
// rotations (Golub and Van Loan, Matrix Computations, section 8.5).
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "oscar_device.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr int kMaxCalibTokens = 4096;

// out[grp] = (1/rows) sum over rows of x_row^T x_row, where the rows of group
// grp are the heads grp*g .. grp*g+g-1 of every token: x is [N][H][128].
template <typename T>
__global__ void __launch_bounds__(256)
cov_kernel(const T* __restrict__ x, int n, int h_total, int g, double* __restrict__ out) {
  const int ti = blockIdx.x >> 3, tj = blockIdx.x & 7, grp = blockIdx.y;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  __shared__ double xi[64][17];
  __shared__ double xj[64][17];
  const int rows = n * g;
  double acc = 0.0;
  for (int r0 = 0; r0 < rows; r0 += 64) {
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      const int rr = e >> 4, c = e & 15, r = r0 + rr;
      double a = 0.0, b = 0.0;
      if (r < rows) {
        const size_t base = (static_cast<size_t>(r / g) * h_total + grp * g + r % g) * kDim;
        a = static_cast<double>(x[base + ti * 16 + c]);
        b = static_cast<double>(x[base + tj * 16 + c]);
      }
      xi[rr][c] = a;
      xj[rr][c] = b;
    }
    __syncthreads();
#pragma unroll 8
    for (int rr = 0; rr < 64; ++rr) acc = fma(xi[rr][ty], xj[rr][tx], acc);
    __syncthreads();
  }
  out[(static_cast<size_t>(grp) * kDim + ti * 16 + ty) * kDim + tj * 16 + tx] = acc / rows;
}

// o[n][h] = sum_{t <= n} softmax_t(q_n . k_t / sqrt(128)) v_t, float64;
// workgroup = (query position n, query head h), 128 threads.
__global__ void __launch_bounds__(128)
calib_attn_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                  int hq, int hkv, double* __restrict__ o) {
  const int n = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int kvh = h / (hq / hkv);
  __shared__ double qs[kDim];
  __shared__ double sc[kMaxCalibTokens];
  __shared__ double red[kDim];
  qs[tid] = static_cast<double>(q[(static_cast<size_t>(n) * hq + h) * kDim + tid]);
  __syncthreads();
  const double inv_sqrt_d = 1.0 / sqrt(static_cast<double>(kDim));
  double mx = -INFINITY;
  for (int t = tid; t <= n; t += kDim) {
    const float4* kr = reinterpret_cast<const float4*>(k + (static_cast<size_t>(t) * hkv + kvh) * kDim);
    double s = 0.0;
    for (int c4 = 0; c4 < kDim / 4; ++c4) {
      const float4 kk = kr[c4];
      s = fma(qs[4 * c4 + 0], static_cast<double>(kk.x), s);
      s = fma(qs[4 * c4 + 1], static_cast<double>(kk.y), s);
      s = fma(qs[4 * c4 + 2], static_cast<double>(kk.z), s);
      s = fma(qs[4 * c4 + 3], static_cast<double>(kk.w), s);
    }
    s *= inv_sqrt_d;
    sc[t] = s;
    mx = fmax(mx, s);
  }
  red[tid] = mx;
  __syncthreads();
  for (int w = 64; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmax(red[tid], red[tid + w]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  double sum = 0.0;
  for (int t = tid; t <= n; t += kDim) {
    const double p = exp(sc[t] - mx);
    sc[t] = p;
    sum += p;
  }
  red[tid] = sum;
  __syncthreads();
  for (int w = 64; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const double total = red[0];
  double acc = 0.0;
  for (int t = 0; t <= n; ++t)
    acc = fma(sc[t], static_cast<double>(v[(static_cast<size_t>(t) * hkv + kvh) * kDim + tid]), acc);
  o[(static_cast<size_t>(n) * hq + h) * kDim + tid] = acc / total;
}

// clip[grp][ch] = percentile_pct of |x_n . R[:, ch]| over n (linear
// interpolation between order statistics); workgroup = (channel, KV head).
__global__ void __launch_bounds__(256)
clip_kernel(const float* __restrict__ x, const double* __restrict__ r, int n, int hkv, double pct,
            float* __restrict__ clip) {
  const int ch = blockIdx.x, grp = blockIdx.y, tid = threadIdx.x;
  __shared__ double vals[kMaxCalibTokens];
  int p2 = 1;
  while (p2 < n) p2 <<= 1;
  const double* rg = r + static_cast<size_t>(grp) * kDim * kDim;
  for (int i = tid; i < p2; i += 256) {
    double y = INFINITY;
    if (i < n) {
      const float* xr = x + (static_cast<size_t>(i) * hkv + grp) * kDim;
      double s = 0.0;
      for (int c = 0; c < kDim; ++c) s = fma(static_cast<double>(xr[c]), rg[c * kDim + ch], s);
      y = fabs(s);
    }
    vals[i] = y;
  }
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= p2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < p2; i += 256) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const double a = vals[i], b = vals[j];
          if ((a > b) == up) {
            vals[i] = b;
            vals[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) {
    const double pos = pct / 100.0 * (n - 1);
    int lo = static_cast<int>(floor(pos));
    if (lo > n - 1) lo = n - 1;
    const int hi = lo + 1 < n ? lo + 1 : n - 1;
    const double t = pos - lo;
    const double a = vals[lo], b = vals[hi];
    const double d = b - a;
    // two-sided form keeps the interpolation monotone and exact at both ends
    const double res = t >= 0.5 ? b - d * (1.0 - t) : a + d * t;
    clip[grp * kDim + ch] = static_cast<float>(res);
  }
}

// ---------------------------------------------------------------- host side

// Cyclic Jacobi eigen-decomposition of a symmetric n x n matrix (row major).
// On return lam holds the eigenvalues and the columns of u the eigenvectors.
void jacobi_eigen(const double* c, int n, std::vector<double>& lam, std::vector<double>& u) {
  std::vector<double> a(c, c + static_cast<size_t>(n) * n);
  u.assign(static_cast<size_t>(n) * n, 0.0);
  for (int i = 0; i < n; ++i) u[i * n + i] = 1.0;
  double frob = 0.0;
  for (double x : a) frob += x * x;
  frob = sqrt(frob);
  for (int sweep = 0; sweep < 60; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) off += a[p * n + q] * a[p * n + q];
    if (sqrt(2.0 * off) <= 1e-15 * frob || off == 0.0) break;
    for (int p = 0; p < n - 1; ++p) {
      for (int q = p + 1; q < n; ++q) {
        const double apq = a[p * n + q];
        if (apq == 0.0) continue;
        const double app = a[p * n + p], aqq = a[q * n + q];
        // rotation angle zeroing a_pq (Golub and Van Loan, sym.schur2)
        const double tau = (aqq - app) / (2.0 * apq);
        const double t = (tau >= 0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
        const double cs = 1.0 / sqrt(1.0 + t * t);
        const double sn = t * cs;
        for (int k = 0; k < n; ++k) {   // columns p, q
          const double akp = a[k * n + p], akq = a[k * n + q];
          a[k * n + p] = cs * akp - sn * akq;
          a[k * n + q] = sn * akp + cs * akq;
        }
        for (int k = 0; k < n; ++k) {   // rows p, q
          const double apk = a[p * n + k], aqk = a[q * n + k];
          a[p * n + k] = cs * apk - sn * aqk;
          a[q * n + k] = sn * apk + cs * aqk;
        }
        a[p * n + q] = a[q * n + p] = 0.0;
        for (int k = 0; k < n; ++k) {
          const double ukp = u[k * n + p], ukq = u[k * n + q];
          u[k * n + p] = cs * ukp - sn * ukq;
          u[k * n + q] = sn * ukp + cs * ukq;
        }
      }
    }
  }
  lam.resize(n);
  for (int i = 0; i < n; ++i) lam[i] = a[i * n + i];
}

int bitrev7(int i) {
  int r = 0;
  for (int b = 0; b < 7; ++b) r |= ((i >> b) & 1) << (6 - b);
  return r;
}

// R = U . H . P for the eigenvectors of c, eigenvalues in descending order,
// each eigenvector signed so that its largest-magnitude entry (lowest index
// on ties) is positive.
void rotation_from_covariance(const double* c, double* r) {
  std::vector<double> lam, u;
  jacobi_eigen(c, kDim, lam, u);
  std::vector<int> order(kDim);
  for (int i = 0; i < kDim; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return lam[x] > lam[y]; });
  std::vector<double> us(static_cast<size_t>(kDim) * kDim);
  for (int j = 0; j < kDim; ++j) {
    const int src = order[j];
    int imax = 0;
    for (int i = 1; i < kDim; ++i)
      if (fabs(u[i * kDim + src]) > fabs(u[imax * kDim + src])) imax = i;
    const double sgn = u[imax * kDim + src] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < kDim; ++i) us[i * kDim + j] = sgn * u[i * kDim + src];
  }
  // (U H)[i][m] = sum_j U[i][j] (-1)^popcount(j & m) / sqrt(128); then column
  // k of R is column bitrev(k) of U H.
  const double hs = 1.0 / sqrt(static_cast<double>(kDim));
  std::vector<double> uh(static_cast<size_t>(kDim) * kDim);
  for (int i = 0; i < kDim; ++i)
    for (int m = 0; m < kDim; ++m) {
      double s = 0.0;
      for (int j = 0; j < kDim; ++j) s += (__builtin_popcount(j & m) & 1) ? -us[i * kDim + j] : us[i * kDim + j];
      uh[i * kDim + m] = s * hs;
    }
  for (int i = 0; i < kDim; ++i)
    for (int k = 0; k < kDim; ++k) r[i * kDim + k] = uh[i * kDim + bitrev7(k)];
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct CalibLayout {
  size_t off_c = 0, off_o = 0, off_r = 0, total = 0;
};

CalibLayout calib_layout(const oscar_dims& d, int n) {
  CalibLayout l;
  const size_t mats = static_cast<size_t>(d.num_kv_heads) * kDim * kDim * sizeof(double);
  l.off_c = 0;
  l.off_o = align256(2 * mats);
  l.off_r = align256(l.off_o + static_cast<size_t>(n) * d.num_q_heads * kDim * sizeof(double));
  l.total = align256(l.off_r + 2 * mats);
  return l;
}

}  // namespace

size_t calibrate_workspace_bytes(const oscar_dims& d, int32_t n_tokens) {
  return calib_layout(d, n_tokens).total;
}

int32_t calibrate_max_tokens() { return kMaxCalibTokens; }

hipError_t run_calibration(const oscar_dims& d, int32_t n, const float* q, const float* k,
                           const float* v, double pct, float* r_k, float* r_v, float* clip_k,
                           float* clip_v, double* r_k_host, double* r_v_host, void* workspace,
                           hipStream_t s) {
  const int hq = d.num_q_heads, hkv = d.num_kv_heads, g = hq / hkv;
  const CalibLayout lay = calib_layout(d, n);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t mat = static_cast<size_t>(kDim) * kDim;
  double* c_q = reinterpret_cast<double*>(ws + lay.off_c);
  double* c_s = c_q + hkv * mat;
  double* o = reinterpret_cast<double*>(ws + lay.off_o);
  double* r64 = reinterpret_cast<double*>(ws + lay.off_r);
  hipError_t e;
  cov_kernel<float><<<dim3(64, hkv), 256, 0, s>>>(q, n, hq, g, c_q);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  calib_attn_kernel<<<dim3(n, hq), 128, 0, s>>>(q, k, v, hq, hkv, o);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  cov_kernel<double><<<dim3(64, hkv), 256, 0, s>>>(o, n, hq, g, c_s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  std::vector<double> cov(2 * hkv * mat), rot(2 * hkv * mat);
  if ((e = hipMemcpyAsync(cov.data(), c_q, cov.size() * sizeof(double), hipMemcpyDeviceToHost, s)) != hipSuccess)
    return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  for (int m = 0; m < 2 * hkv; ++m) rotation_from_covariance(cov.data() + m * mat, rot.data() + m * mat);
  if (r_k_host) memcpy(r_k_host, rot.data(), hkv * mat * sizeof(double));
  if (r_v_host) memcpy(r_v_host, rot.data() + hkv * mat, hkv * mat * sizeof(double));
  if ((e = hipMemcpyAsync(r64, rot.data(), rot.size() * sizeof(double), hipMemcpyHostToDevice, s)) != hipSuccess)
    return e;
  clip_kernel<<<dim3(kDim, hkv), 256, 0, s>>>(k, r64, n, hkv, pct, clip_k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  clip_kernel<<<dim3(kDim, hkv), 256, 0, s>>>(v, r64 + hkv * mat, n, hkv, pct, clip_v);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  std::vector<float> r32(rot.size());
  for (size_t i = 0; i < rot.size(); ++i) r32[i] = static_cast<float>(rot[i]);
  if ((e = hipMemcpyAsync(r_k, r32.data(), hkv * mat * sizeof(float), hipMemcpyHostToDevice, s)) != hipSuccess)
    return e;
  if ((e = hipMemcpyAsync(r_v, r32.data() + hkv * mat, hkv * mat * sizeof(float), hipMemcpyHostToDevice, s)) !=
      hipSuccess)
    return e;
  return hipStreamSynchronize(s);
}

}  // namespace oscar
