// Host-side declarations shared between the OSCAR entry points and the
// kernel launchers.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/oscar.h"

namespace oscar {

// bf16 sink/recent partials per (request, query head): the sink and four
// quarters of the recent ring.
constexpr int kBf16Parts = 5;
// Upper bound on the history splits of one request.
constexpr int kMaxSplits = 251;
// Smallest history split, in pages.
constexpr int kMinSplitPages = 4;
// The history split schedule aims by default for the workgroups the
// matrix-core history kernel keeps resident on the device's SIMDs (4 per
// compute unit, read from the device; hist_default_target), so the splits
// run in one round.
// Default target of the all-bf16 baseline (two one-wave workgroups per
// SIMD of a 256-CU MI355X; halved for query groups wider than four heads).
constexpr int kDefaultTargetWg = 2048;
// Largest settable target (bounds the workspace).
constexpr int kMaxTargetWg = 8192;

// Workspace layout of one decode call (offsets in bytes, 256-aligned).
//
// History splits are scheduled on the device (the query-rotation kernel
// reads the lengths): the batch's history pages are cut into splits of at
// most q pages, each request getting ceil(pages / q) equal ones, numbered
// 0 .. n_splits-1 across the batch.  `slots` bounds n_splits; the history
// kernels launch slots x Hkv workgroups and the unused ones exit at once.
// The split tables and partials are sized for ceil(kMaxTargetWg / Hkv) + B
// splits whatever the target, so the offsets depend only on (dims, B).
struct WsLayout {
  int32_t target = 1;           // splits per KV head the schedule aims for
  int32_t slots = 1;            // upper bound on splits per KV head
  size_t off_qrot = 0;          // float [B][Hq][128]: R_K-rotated query * log2(e)/sqrt(128)
  size_t off_qsum = 0;          // float [B][Hq][4]: per-group sums of that query
  size_t off_qpack = 0;         // matrix-core operands, kQPackBytes per (b, kv head)
  size_t off_sched = 0;         // int32 [1 + 3 * slots]: n_splits, then {request, page0, page1}
  size_t off_req = 0;           // int32 [B][2]: {first split, split count}
  size_t off_ho = 0;            // float [slots][Hq][128]: history partial outputs (rotated)
  size_t off_hlse = 0;          // float [slots][Hq]: history partial log-sum-exp (natural log)
  size_t off_bo = 0;            // float [B][Hq][5][128]: bf16 partial outputs
  size_t off_blse = 0;          // float [B][Hq][5]
  size_t total = 0;
};

// Matrix-core query operands of one (request, KV head): for each channel
// half (64 channels) and lane group, 32 rows x 16 int8 limb bytes; then the
// same for the query times the Lloyd-Max high-bit weight ratio (written for
// that codebook only); then per-head dequantization scales.
constexpr int kQPackRows = 32;
constexpr size_t kQPackOperandBytes = 2 * 4 * kQPackRows * 16;  // 4096
constexpr size_t kQPackScaleOffset = 2 * kQPackOperandBytes;
constexpr size_t kQPackBytes = kQPackScaleOffset + 256;

// target_wg: history workgroups the call's split schedule aims for (> 0);
// the offsets and total do not depend on it.
// Record `msg` as the calling thread's last error (oscar_last_error) and
// return `code`.
int set_error(int code, const char* msg);

WsLayout workspace_layout(const oscar_dims& d, int32_t batch, int32_t max_seq_len, int target_wg);

// Float32 levels (ascending) and decision thresholds of a codebook
// (OSCAR_CODEBOOK_*); nullptr for an unknown one.
struct Codebook {
  float lev[4];
  float thr[3];
};
const Codebook* codebook_of(int32_t codebook);

struct DemoteArgs {
  const float* r;        // [Hkv][128][128], K or V per blockIdx.z
  const float* clip;
  uint8_t* pages;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t hkv;
  int32_t codebook;      // OSCAR_CODEBOOK_*
  float thr;             // Lloyd-Max: the positive decision threshold
};

// Everything one decode step's demotion reads and writes.
struct DemoteStep {
  DemoteArgs kk, vv;
  const int32_t* seq_lens;
  uint16_t* sink_k;
  uint16_t* sink_v;
  uint16_t* recent_k;
  uint16_t* recent_v;
  const uint16_t* k_new;
  const uint16_t* v_new;
};

DemoteStep make_demote_step(const oscar_dims& d, const oscar_rotation& rot, const oscar_cache& c,
                            const uint16_t* k_new, const uint16_t* v_new);
hipError_t launch_demote(const oscar_dims& d, const oscar_rotation& rot, const oscar_cache& c,
                         const uint16_t* k_new, const uint16_t* v_new, hipStream_t s);
hipError_t launch_fill(const oscar_dims& d, const oscar_rotation& rot, const oscar_cache& c,
                       int32_t request, int32_t hist_begin, int32_t n_tokens,
                       const uint16_t* k_tokens, const uint16_t* v_tokens, hipStream_t s);
hipError_t launch_read_history(const oscar_dims& d, const oscar_cache& c, int32_t request, int32_t hist_begin,
                               int32_t n_tokens, float* k_out, float* v_out, hipStream_t s);

struct DecodeArgs {
  const oscar_dims* dims;
  const oscar_rotation* rot;
  const oscar_cache* cache;
  const uint16_t* q;
  uint8_t* ws;
  WsLayout lay;
  hipEvent_t ev_start = nullptr;   // when both set, the history kernel is launched
  hipEvent_t ev_stop = nullptr;    // with these as its start/stop timestamps
  unsigned long long* clock_trace = nullptr;   // when set, the history kernel's first
                                               // workgroup records its clock counters
  const DemoteStep* demote = nullptr;   // when set, the prologue launch also demotes
  // History split slots per KV head the matrix-core launch holds, and the
  // target the call's split schedule aims for (history_launch_slots).
  int32_t hist_slots = 0;
  int32_t sched_target = 0;
};

// The history split slots (per KV head) a decode call launches, and the
// schedule target that keeps the schedule inside them.  The schedule makes
// at most max(target, batch) splits, and at most ceil(pages / kMinSplitPages)
// per request, pages from max_seq_len (the API requires max_seq_len >= every
// length).  The launch holds n = max(batch, min(max(t, batch),
// batch * ceil(pages / kMinSplitPages))) slots, t the layout's target; the
// schedule aims for min(t, n), which gives the same schedule as t whenever
// the lengths respect max_seq_len, and at most n splits even when they do
// not.  (The workspace's t + batch slots, launched whole, made a 1 x 100K
// launch dispatch about twice the workgroups that had work, which cost it
// 1.5 us.)
void history_launch_slots(const WsLayout& lay, int32_t batch, int32_t max_seq_len, int32_t* slots,
                          int32_t* sched_target);

hipError_t launch_qrot(const DecodeArgs& a, hipStream_t s);
hipError_t launch_hist_valu(const DecodeArgs& a, hipStream_t s);
hipError_t launch_hist_mfma(const DecodeArgs& a, hipStream_t s);
bool hist_mfma_supported(const oscar_dims& d);
// Workgroups of the matrix-core history kernel for dims resident on `simds` SIMDs.
int hist_default_target(const oscar_dims& d, int simds);
hipError_t launch_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_merge(const oscar_dims& d, const oscar_rotation& rot, int32_t batch,
                        const uint8_t* ws, const WsLayout& lay, float* out, float* lse_out,
                        hipStream_t s);

// ---- all-bf16 baseline (baseline_bf16.hip)
struct BaseLayout {
  int32_t target = 1;
  int32_t slots = 1;
  size_t off_sched = 0;   // int32 [1 + 3 cap]
  size_t off_req = 0;     // int32 [B][2]
  size_t off_ho = 0;      // float [cap][Hq][128]
  size_t off_hlse = 0;    // float [cap][Hq]
  size_t total = 0;
};
BaseLayout base_layout(const oscar_dims& d, int32_t batch, int target_wg);
hipError_t launch_base_decode(const oscar_dims& d, const oscar_bf16_cache& c, const uint16_t* q, uint8_t* ws,
                              const BaseLayout& lay, float* out, float* lse_out, hipStream_t s, hipEvent_t ev0,
                              hipEvent_t ev1);
hipError_t launch_base_fill(const oscar_dims& d, const oscar_bf16_cache& c, int32_t request, int32_t pos_begin,
                            int32_t n_tokens, const uint16_t* k_tokens, const uint16_t* v_tokens, hipStream_t s);
hipError_t launch_base_append(const oscar_dims& d, const oscar_bf16_cache& c, const uint16_t* k_new,
                              const uint16_t* v_new, hipStream_t s);

size_t calibrate_workspace_bytes(const oscar_dims& d, int32_t n_tokens);
int32_t calibrate_max_tokens();
hipError_t run_calibration(const oscar_dims& d, int32_t n, const float* q, const float* k,
                           const float* v, double pct, float* r_k, float* r_v, float* clip_k,
                           float* clip_v, double* r_k_host, double* r_v_host, void* workspace,
                           hipStream_t s);

}  // namespace oscar
