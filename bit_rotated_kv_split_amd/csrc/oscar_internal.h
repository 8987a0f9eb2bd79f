// Host-side declarations shared between the OSCAR entry points and the
// kernel launchers.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/oscar.h"

namespace oscar {

// Partials per (request, query head): S history splits, then the bf16
// sink/recent chunks (the sink and four quarters of the ring).
constexpr int kBf16Parts = 5;
constexpr int kMaxSplits = 251;
constexpr int kMaxParts = kMaxSplits + kBf16Parts;

// Workspace layout of one decode call (offsets in bytes, 256-aligned).
struct WsLayout {
  int32_t splits = 1;           // history splits S
  int32_t parts = 1 + kBf16Parts;
  int32_t pages_per_split = 0;  // pages one split covers
  size_t off_qrot = 0;          // float [B][Hq][128]: R_K-rotated query * log2(e)/sqrt(128)
  size_t off_qsum = 0;          // float [B][Hq][4]: per-group sums of that query
  size_t off_qpack = 0;         // matrix-core operands, kQPackBytes per (b, kv head)
  size_t off_po = 0;            // float [B][Hq][parts][128] partial outputs
  size_t off_plse = 0;          // float [B][Hq][parts] partial log-sum-exp (natural log)
  size_t total = 0;
};

// Matrix-core query operand of one (request, KV head): for each channel half
// (64 channels) and lane group, 32 rows x 16 int8 limb bytes, then per-head
// dequantization scales.
constexpr int kQPackRows = 32;
constexpr size_t kQPackOperandBytes = 2 * 4 * kQPackRows * 16;  // 4096
constexpr size_t kQPackBytes = kQPackOperandBytes + 256;

WsLayout workspace_layout(const oscar_dims& d, int32_t batch, int32_t max_seq_len);

struct DemoteArgs {
  const float* r;        // [Hkv][128][128], K or V per blockIdx.z
  const float* clip;
  uint8_t* pages;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t hkv;
};

hipError_t launch_demote(const oscar_dims& d, const oscar_rotation& rot, const oscar_cache& c,
                         const uint16_t* k_new, const uint16_t* v_new, hipStream_t s);
hipError_t launch_fill(const oscar_dims& d, const oscar_rotation& rot, const oscar_cache& c,
                       int32_t request, int32_t hist_begin, int32_t n_tokens,
                       const uint16_t* k_tokens, const uint16_t* v_tokens, hipStream_t s);

struct DecodeArgs {
  const oscar_dims* dims;
  const oscar_rotation* rot;
  const oscar_cache* cache;
  const uint16_t* q;
  uint8_t* ws;
  WsLayout lay;
  hipEvent_t ev_start = nullptr;   // when both set, the history kernel is launched
  hipEvent_t ev_stop = nullptr;    // with these as its start/stop timestamps
};

hipError_t launch_qrot(const DecodeArgs& a, hipStream_t s);
hipError_t launch_hist_valu(const DecodeArgs& a, hipStream_t s);
hipError_t launch_hist_mfma(const DecodeArgs& a, hipStream_t s);
bool hist_mfma_supported(const oscar_dims& d);
hipError_t launch_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_merge(const oscar_dims& d, const oscar_rotation& rot, int32_t batch,
                        const uint8_t* ws, const WsLayout& lay, float* out, float* lse_out,
                        hipStream_t s);

size_t calibrate_workspace_bytes(const oscar_dims& d, int32_t n_tokens);
int32_t calibrate_max_tokens();
hipError_t run_calibration(const oscar_dims& d, int32_t n, const float* q, const float* k,
                           const float* v, double pct, float* r_k, float* r_v, float* clip_k,
                           float* clip_v, double* r_k_host, double* r_v_host, void* workspace,
                           hipStream_t s);

}  // namespace oscar
