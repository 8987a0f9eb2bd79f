// Device helpers shared by the OSCAR HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int kDim = 128;        // head dimension
constexpr int kPage = 64;        // history slots per page
constexpr int kSink = 64;        // bf16 sink tokens
constexpr int kRecent = 256;     // bf16 recent window
constexpr int kBf16Tokens = kSink + kRecent;
constexpr int kKWordsBytes = 2048;   // key words of one block
constexpr int kCodesBytes = 4096;    // key + value words of one block

__host__ __device__ constexpr int block_bytes(int G) { return kCodesBytes + 512 * (kDim / G); }

// Stored form of a word of sixteen 2-bit codes (code i at bits 2i, 2i+1):
// the code in the top two bits of each byte (i % 4 == 3) is kept XOR 2, so
// a stored word is the plain packing XOR 0x80808080.  Masked in place
// (word & 0xC0C0C0C0), that field then reads as the signed byte
// 64 (code - 2): linear in the code, which lets the matrix-core kernel take
// it with one AND instead of a shift and an AND.
constexpr uint32_t kTopFieldFlip = 0x80808080u;

// Stored bits of code c at position i of a word.
__host__ __device__ constexpr uint32_t code_bits(uint32_t c, int i) {
  return (c ^ ((i & 3) == 3 ? 2u : 0u)) << (2 * i);
}

// Position of slot t in the key-word rows and in the scale/zero tables:
// the order in which the matrix-core history kernel's lanes consume tokens.
__host__ __device__ __forceinline__ int qk_order(int t) {
  return 16 * (t >> 4) + 4 * (t & 3) + ((t >> 2) & 3);
}

// Word index (within the value words) of channel c, token group w (16 slots).
__host__ __device__ __forceinline__ int v_word_index(int c, int w) {
  return (c >> 6) * 256 + (w * 16 + (c & 15)) * 4 + ((c >> 4) & 3);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(f32_to_bf16_rne(x)); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

struct WaveMax {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct WaveAdd {
  __device__ float operator()(float a, float b) const { return a + b; }
};

// Reduction over the whole wave: DPP steps inside each 16-lane row (every
// lane of a row ends with the row's result), then the four rows read back
// with v_readlane.  The result is uniform.  Much shorter than a chain of
// cross-lane permutes through LDS.
template <typename Op>
__device__ __forceinline__ float wave_reduce_dpp(float v, Op op) {
  int x = __float_as_int(v);
  x = __float_as_int(op(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false))));
  x = __float_as_int(op(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false))));
  x = __float_as_int(op(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false))));
  x = __float_as_int(op(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false))));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(x, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(x, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(x, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(x, 48));
  return op(op(r0, r1), op(r2, r3));
}

// log2(e) / sqrt(128): scores are kept in base-2 units inside the kernels.
constexpr float kScoreScaleLog2 = 1.4426950408889634f * 0.08838834764831845f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

}  // namespace oscar
