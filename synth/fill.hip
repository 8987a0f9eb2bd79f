// GPU twin of synth/gen.py: the same counter-based SplitMix64 draws and the
// same Irwin-Hall(12) normal, writing bf16 K or V tokens straight into device
// buffers.  Random draws and layout only; none of the method's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float normal_f32(uint64_t key, uint64_t idx) {
  int64_t total = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const uint64_t r = mix64(key + (idx * 3 + j + 1) * kGolden);
#pragma unroll
    for (int k = 0; k < 4; ++k) total += static_cast<int64_t>((r >> (16 * k)) & 0xFFFF);
  }
  return static_cast<float>(total - 393210) * 1.52587890625e-05f;   // 2^-16, exact
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// dst element of (token t, head h, channel c) = dst[t*stride_t + h*stride_h + c]
__global__ void fill_kernel(uint16_t* __restrict__ dst, int32_t n_tok, int32_t hkv, int64_t stride_t,
                            int64_t stride_h, uint64_t key, uint32_t src, int32_t pos0,
                            const float* __restrict__ scale) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(n_tok) * hkv * 128;
  if (i >= total) return;
  const int c = static_cast<int>(i & 127);
  const int h = static_cast<int>((i >> 7) % hkv);
  const int t = static_cast<int>((i >> 7) / hkv);
  const uint64_t base = (static_cast<uint64_t>(src) * 64 + static_cast<uint64_t>(h)) << 21;
  const uint64_t idx = ((base + static_cast<uint64_t>(pos0 + t)) << 7) + static_cast<uint64_t>(c);
  const float x = normal_f32(key, idx) * scale[h * 128 + c];
  dst[t * stride_t + h * stride_h + c] = bf16_rne(x);
}

}  // namespace

extern "C" int synth_fill_kv(void* dst, int32_t n_tok, int32_t hkv, int64_t stride_t, int64_t stride_h,
                             uint64_t key, uint32_t src, int32_t pos0, const float* scale,
                             void* stream) {
  if (n_tok <= 0) return 0;
  if (dst == nullptr || scale == nullptr || hkv <= 0 || hkv > 64 || pos0 < 0 ||
      static_cast<int64_t>(pos0) + n_tok > (1 << 21))
    return 1;
  const int64_t total = static_cast<int64_t>(n_tok) * hkv * 128;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return 1;
  fill_kernel<<<static_cast<unsigned>(blocks), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<uint16_t*>(dst), n_tok, hkv, stride_t, stride_h, key, src, pos0, scale);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
