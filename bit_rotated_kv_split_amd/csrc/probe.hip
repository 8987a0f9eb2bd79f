// HBM read-bandwidth probe (oscar_probe_read): the ceiling the history
// kernel's roofline fraction is compared against on the same device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/oscar_probe.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
// workgroups of one pass: eight per compute unit of a 256-CU device, so
// every SIMD holds several waves with loads in flight
constexpr int kProbeBlocks = 2048;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

template <bool NT>
__device__ __forceinline__ v4u load16(const v4u* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT>
__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const v4u* __restrict__ p, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kProbeThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    v4u v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = load16<NT>(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const v4u v = load16<NT>(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kProbeMagic) sink[0] = acc;
}

// Block-streaming form: one wave per workgroup reads its own contiguous
// share in 4 KB blocks (four 16-byte loads per lane, 1 KB per load across
// the wave), with kBlocksInFlight blocks in flight: the access pattern of
// the history kernel's page loads without its arithmetic.
constexpr int kBlockBytes = 4096;
constexpr int kBlocksInFlight = 4;

template <bool NT>
__global__ void __launch_bounds__(64) read_blocks_kernel(const v4u* __restrict__ p, size_t blocks_per_wave,
                                                         uint32_t* __restrict__ sink) {
  constexpr int kPerBlock = kBlockBytes / 16;   // 16-byte words of a block
  const int lane = threadIdx.x;
  const v4u* base = p + static_cast<size_t>(blockIdx.x) * blocks_per_wave * kPerBlock;
  uint32_t acc = 0;
  size_t blk = 0;
  for (; blk + kBlocksInFlight <= blocks_per_wave; blk += kBlocksInFlight) {
    v4u v[kBlocksInFlight][4];
#pragma unroll
    for (int f = 0; f < kBlocksInFlight; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[f][j] = load16<NT>(base + (blk + f) * kPerBlock + 64 * j + lane);
#pragma unroll
    for (int f = 0; f < kBlocksInFlight; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= v[f][j].x ^ v[f][j].y ^ v[f][j].z ^ v[f][j].w;
  }
  for (; blk < blocks_per_wave; ++blk)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4u v = load16<NT>(base + blk * kPerBlock + 64 * j + lane);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  if (acc == kProbeMagic) sink[0] = acc;
}

}  // namespace
}  // namespace oscar

extern "C" int oscar_probe_read_blocks(const void* buf, size_t bytes, int32_t nontemporal, int32_t waves,
                                       uint32_t* sink, void* stream) {
  using namespace oscar;
  if (buf == nullptr || sink == nullptr) return set_error(OSCAR_EINVAL, "probe buffer or sink is NULL");
  if (waves <= 0) return set_error(OSCAR_EINVAL, "waves must be positive");
  if ((reinterpret_cast<uintptr_t>(buf) & 15) || bytes % (static_cast<size_t>(waves) * kBlockBytes) != 0)
    return set_error(OSCAR_EINVAL, "probe buffer must be 16-byte aligned and a multiple of waves x 4096 bytes");
  if (bytes == 0) return OSCAR_OK;
  const size_t per_wave = bytes / (static_cast<size_t>(waves) * kBlockBytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const v4u* p = static_cast<const v4u*>(buf);
  if (nontemporal)
    read_blocks_kernel<true><<<waves, 64, 0, s>>>(p, per_wave, sink);
  else
    read_blocks_kernel<false><<<waves, 64, 0, s>>>(p, per_wave, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(OSCAR_EHIP, hipGetErrorString(e));
  return OSCAR_OK;
}

extern "C" int oscar_probe_read(const void* buf, size_t bytes, int32_t nontemporal, uint32_t* sink,
                                void* stream) {
  using namespace oscar;
  if (buf == nullptr || sink == nullptr) return set_error(OSCAR_EINVAL, "probe buffer or sink is NULL");
  if ((reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15))
    return set_error(OSCAR_EINVAL, "probe buffer must be 16-byte aligned and a multiple of 16 bytes");
  if (bytes == 0) return OSCAR_OK;
  const size_t n16 = bytes / 16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const v4u* p = static_cast<const v4u*>(buf);
  if (nontemporal)
    read_probe_kernel<true><<<kProbeBlocks, kProbeThreads, 0, s>>>(p, n16, sink);
  else
    read_probe_kernel<false><<<kProbeBlocks, kProbeThreads, 0, s>>>(p, n16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(OSCAR_EHIP, hipGetErrorString(e));
  return OSCAR_OK;
}
