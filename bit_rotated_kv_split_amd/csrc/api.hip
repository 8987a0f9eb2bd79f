// C ABI entry points of the OSCAR decode path: argument checks, workspace
// layout and launch order.  Every compute step runs in the HIP kernels of
// demote.hip, decode.hip and decode_mfma.hip.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>

#include "oscar_device.h"
#include "oscar_internal.h"

namespace oscar {
namespace {

thread_local std::string g_error;
// Compute units of each device, read once from the device and kept (an
// immutable hardware attribute, not a setting; 0 = not read yet).
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(OSCAR_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int check_dims(const oscar_dims* d) {
  if (d == nullptr) return fail(OSCAR_EINVAL, "dims is NULL");
  if (d->head_dim != kDim) return fail(OSCAR_EUNSUPPORTED, "head_dim %d unsupported (128 only)", d->head_dim);
  if (d->page_size != kPage) return fail(OSCAR_EUNSUPPORTED, "page_size %d unsupported (64 only)", d->page_size);
  if (d->sink_len != kSink || d->recent_len != kRecent)
    return fail(OSCAR_EUNSUPPORTED, "sink/recent %d/%d unsupported (64/256 only)", d->sink_len, d->recent_len);
  if (d->group_size != 32 && d->group_size != 64 && d->group_size != 128)
    return fail(OSCAR_EUNSUPPORTED, "group_size %d unsupported (32, 64, 128)", d->group_size);
  if (d->num_kv_heads <= 0 || d->num_q_heads <= 0)
    return fail(OSCAR_EINVAL, "head counts must be positive (%d q, %d kv)", d->num_q_heads, d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(OSCAR_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", d->num_q_heads, d->num_kv_heads);
  const int g = d->num_q_heads / d->num_kv_heads;
  if (g > 8) return fail(OSCAR_EUNSUPPORTED, "query heads per KV head %d unsupported (<= 8)", g);
  if (codebook_of(d->codebook) == nullptr)
    return fail(OSCAR_EUNSUPPORTED, "codebook %d unsupported (0 uniform, 1 Lloyd-Max)", d->codebook);
  return OSCAR_OK;
}

int check_rot(const oscar_rotation* r) {
  if (r == nullptr) return fail(OSCAR_EINVAL, "rotation is NULL");
  if (!r->r_k || !r->r_v || !r->clip_k || !r->clip_v)
    return fail(OSCAR_EINVAL, "rotation has a NULL pointer");
  return OSCAR_OK;
}

int check_cache(const oscar_cache* c, bool need_pages) {
  if (c == nullptr) return fail(OSCAR_EINVAL, "cache is NULL");
  if (c->batch < 0) return fail(OSCAR_EINVAL, "batch %d < 0", c->batch);
  if (c->batch == 0) return OSCAR_OK;
  if (!c->sink_k || !c->sink_v || !c->recent_k || !c->recent_v || !c->seq_lens)
    return fail(OSCAR_EINVAL, "cache has a NULL sink/recent/seq_lens pointer");
  if (need_pages) {
    if (!c->pages || !c->page_table) return fail(OSCAR_EINVAL, "cache has a NULL pages/page_table pointer");
    if (c->max_pages_per_req <= 0 || c->n_pages <= 0)
      return fail(OSCAR_EINVAL, "max_pages_per_req %d / n_pages %lld must be positive",
                  c->max_pages_per_req, static_cast<long long>(c->n_pages));
  }
  return OSCAR_OK;
}

int check_bf16_cache(const oscar_bf16_cache* c) {
  if (c == nullptr) return fail(OSCAR_EINVAL, "cache is NULL");
  if (c->batch < 0) return fail(OSCAR_EINVAL, "batch %d < 0", c->batch);
  if (c->batch == 0) return OSCAR_OK;
  if (!c->pages || !c->page_table || !c->seq_lens)
    return fail(OSCAR_EINVAL, "bf16 cache has a NULL pages/page_table/seq_lens pointer");
  if (c->max_pages_per_req <= 0 || c->n_pages <= 0)
    return fail(OSCAR_EINVAL, "max_pages_per_req %d / n_pages %lld must be positive", c->max_pages_per_req,
                static_cast<long long>(c->n_pages));
  return OSCAR_OK;
}

// SIMDs (4 per compute unit) of the current device.
int current_device_simds(int* simds) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "no current HIP device to size the default history target");
  int cus = dev >= 0 && dev < kMaxDevices ? g_device_cus[dev].load(std::memory_order_relaxed) : 0;
  if (cus == 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(OSCAR_EHIP, "compute unit count of device %d: %s", dev, hipGetErrorString(e));
    if (cus <= 0) return fail(OSCAR_EHIP, "device %d reports %d compute units", dev, cus);
    if (dev >= 0 && dev < kMaxDevices) g_device_cus[dev].store(cus, std::memory_order_relaxed);
  }
  *simds = 4 * cus;
  return OSCAR_OK;
}

// Per-call options, validated, with the default target resolved for dims
// when `need_target` (the split schedule is built in this call).
struct CallOpts {
  int kernel = 0;
  int target_wg = 0;
  hipEvent_t ev_start = nullptr;
  hipEvent_t ev_stop = nullptr;
  unsigned long long* clock_trace = nullptr;
};

// The default target when none was given: the resident workgroups of the
// history kernel on the current device (the bf16 baseline keeps a fixed
// default).
int resolve_target(const oscar_dims& d, bool bf16_baseline, CallOpts* c) {
  if (c->target_wg != 0) return OSCAR_OK;
  if (bf16_baseline) {
    c->target_wg = d.num_q_heads / d.num_kv_heads > 4 ? kDefaultTargetWg / 2 : kDefaultTargetWg;
    return OSCAR_OK;
  }
  int simds = 0;
  const int rc = current_device_simds(&simds);
  if (rc) return rc;
  c->target_wg = std::min(hist_default_target(d, simds), kMaxTargetWg);
  return OSCAR_OK;
}

int resolve_opts(const oscar_dims& d, const oscar_decode_options* o, bool need_target, bool bf16_baseline,
                 CallOpts* out) {
  CallOpts c;
  if (o != nullptr) {
    if (o->history_kernel < 0 || o->history_kernel > 2)
      return fail(OSCAR_EINVAL, "history_kernel %d invalid (0 default, 1 vector-ALU, 2 matrix-core)",
                  o->history_kernel);
    if (bf16_baseline && o->history_kernel != 0)
      return fail(OSCAR_EINVAL, "the bf16 baseline has one history kernel (history_kernel must be 0)");
    if (o->history_target < 0 || o->history_target > kMaxTargetWg)
      return fail(OSCAR_EINVAL, "history_target %d outside 0..%d", o->history_target, kMaxTargetWg);
    c.kernel = o->history_kernel;
    c.target_wg = o->history_target;
    if (o->history_start_event != nullptr && o->history_stop_event != nullptr) {
      c.ev_start = static_cast<hipEvent_t>(o->history_start_event);
      c.ev_stop = static_cast<hipEvent_t>(o->history_stop_event);
    }
    c.clock_trace = reinterpret_cast<unsigned long long*>(o->history_clock_trace);
  }
  if (c.kernel == 2 && !hist_mfma_supported(d))
    return fail(OSCAR_EUNSUPPORTED, "matrix-core history kernel does not support these dims");
  *out = c;
  return need_target ? resolve_target(d, bf16_baseline, out) : OSCAR_OK;
}

bool use_mfma(const oscar_dims& d, const CallOpts& c) {
  return c.kernel == 2 || (c.kernel == 0 && hist_mfma_supported(d));
}

int pages_for(int32_t max_seq_len) {
  const int n_hist = max_seq_len > kBf16Tokens ? max_seq_len - kBf16Tokens : 0;
  return (n_hist + kPage - 1) / kPage;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

namespace {

// Workspace of oscar_decode_step_noalloc: a device array of this library's
// code object, so that call needs no allocation.  Each device the library
// is loaded on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: kernels
// and copies get the address hipGetSymbolAddress returns for the current
// device (scratch_address).
static __device__ __align__(256) uint8_t scratch[OSCAR_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "no current HIP device for the no-allocation scratch");
  if (dev < 0 || dev >= kMaxDevices) return fail(OSCAR_EUNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "device address of the no-allocation scratch");
    if (p == nullptr) return fail(OSCAR_EHIP, "device address of the no-allocation scratch is NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return OSCAR_OK;
}

}  // namespace

void history_launch_slots(const WsLayout& lay, int32_t batch, int32_t max_seq_len, int32_t* slots,
                          int32_t* sched_target) {
  const long long pages = pages_for(max_seq_len);
  const long long per_req = (pages + kMinSplitPages - 1) / kMinSplitPages;
  const long long b = batch;
  const long long t = lay.target;
  const long long n = std::max(b, std::min(std::max(t, b), per_req * b));
  *slots = static_cast<int32_t>(std::min<long long>(n, lay.slots));
  *sched_target = static_cast<int32_t>(std::min(t, n));
}

WsLayout workspace_layout(const oscar_dims& d, int32_t batch, int32_t max_seq_len, int target_wg) {
  (void)max_seq_len;
  WsLayout w;
  // the schedule of one call: about target_wg history workgroups (by
  // default as many as the history kernel keeps resident)
  const int t = (std::max(target_wg, 1) + d.num_kv_heads - 1) / d.num_kv_heads;
  w.target = t;
  w.slots = t + batch;
  // storage is sized for the largest target, so the layout (and the
  // merge's view of it) does not depend on the current setting
  const size_t cap = static_cast<size_t>((kMaxTargetWg + d.num_kv_heads - 1) / d.num_kv_heads) + batch;
  const size_t heads = static_cast<size_t>(batch) * d.num_q_heads;
  size_t off = 0;
  w.off_qrot = off;
  off = align256(off + heads * kDim * sizeof(float));
  w.off_qsum = off;
  off = align256(off + heads * 4 * sizeof(float));
  w.off_qpack = off;
  off = align256(off + static_cast<size_t>(batch) * d.num_kv_heads * kQPackBytes);
  w.off_sched = off;
  off = align256(off + (1 + 3 * cap) * sizeof(int32_t));
  w.off_req = off;
  off = align256(off + 2 * static_cast<size_t>(batch) * sizeof(int32_t));
  w.off_ho = off;
  off = align256(off + cap * d.num_q_heads * kDim * sizeof(float));
  w.off_hlse = off;
  off = align256(off + cap * d.num_q_heads * sizeof(float));
  w.off_bo = off;
  off = align256(off + heads * kBf16Parts * kDim * sizeof(float));
  w.off_blse = off;
  off = align256(off + heads * kBf16Parts * sizeof(float));
  w.total = off;
  return w;
}

}  // namespace oscar

using namespace oscar;

extern "C" {

size_t oscar_block_bytes(int32_t group_size) {
  if (group_size != 32 && group_size != 64 && group_size != 128) return 0;
  return static_cast<size_t>(block_bytes(group_size));
}

const char* oscar_last_error(void) { return g_error.c_str(); }

int32_t oscar_calibrate_max_tokens(void) { return calibrate_max_tokens(); }

size_t oscar_calibrate_workspace_bytes(const oscar_dims* dims, int32_t n_tokens) {
  if (check_dims(dims) || n_tokens < 2 || n_tokens > calibrate_max_tokens()) return 0;
  return calibrate_workspace_bytes(*dims, n_tokens);
}

int oscar_calibrate(const oscar_dims* dims, int32_t n_tokens, const float* q, const float* k,
                    const float* v, double clip_percentile, float* r_k, float* r_v, float* clip_k,
                    float* clip_v, double* r_k_host, double* r_v_host, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims))) return rc;
  if (n_tokens < 2 || n_tokens > calibrate_max_tokens())
    return fail(OSCAR_EUNSUPPORTED, "n_tokens %d outside 2..%d", n_tokens, calibrate_max_tokens());
  if (!(clip_percentile > 0.0 && clip_percentile <= 100.0))
    return fail(OSCAR_EINVAL, "clip_percentile %g outside (0, 100]", clip_percentile);
  if (!q || !k || !v || !r_k || !r_v || !clip_k || !clip_v || !workspace)
    return fail(OSCAR_EINVAL, "calibration has a NULL device pointer");
  if (workspace_bytes < calibrate_workspace_bytes(*dims, n_tokens))
    return fail(OSCAR_EINVAL, "workspace %zu bytes < %zu required", workspace_bytes,
                calibrate_workspace_bytes(*dims, n_tokens));
  const hipError_t e = run_calibration(*dims, n_tokens, q, k, v, clip_percentile, r_k, r_v, clip_k,
                                       clip_v, r_k_host, r_v_host, workspace,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "calibration");
  return OSCAR_OK;
}

int oscar_history_kernel_for(const oscar_dims* dims, const oscar_decode_options* options) {
  g_error.clear();
  CallOpts c;
  if (check_dims(dims) || resolve_opts(*dims, options, false, false, &c)) return -1;
  return use_mfma(*dims, c) ? 2 : 1;
}

int oscar_kv_demote(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                    const uint16_t* k_new, const uint16_t* v_new, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_rot(rot)) || (rc = check_cache(cache, true))) return rc;
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(OSCAR_EINVAL, "k_new and v_new must both be set or both be NULL");
  if (cache->batch == 0) return OSCAR_OK;
  const hipError_t e = launch_demote(*dims, *rot, *cache, k_new, v_new, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "demote launch");
  return OSCAR_OK;
}

int oscar_kv_fill_history(const oscar_dims* dims, const oscar_rotation* rot,
                          const oscar_cache* cache, int32_t request, int32_t hist_begin,
                          int32_t n_tokens, const uint16_t* k_tokens, const uint16_t* v_tokens,
                          void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_rot(rot)) || (rc = check_cache(cache, true))) return rc;
  if (request < 0 || request >= cache->batch)
    return fail(OSCAR_EINVAL, "request %d outside batch %d", request, cache->batch);
  if (hist_begin < 0 || n_tokens < 0)
    return fail(OSCAR_EINVAL, "hist_begin %d / n_tokens %d must be >= 0", hist_begin, n_tokens);
  if (n_tokens == 0) return OSCAR_OK;
  if (k_tokens == nullptr || v_tokens == nullptr) return fail(OSCAR_EINVAL, "token pointers are NULL");
  const int64_t last_page = (static_cast<int64_t>(hist_begin) + n_tokens - 1) / kPage;
  if (last_page >= cache->max_pages_per_req)
    return fail(OSCAR_EINVAL, "history index %lld beyond max_pages_per_req %d",
                static_cast<long long>(hist_begin) + n_tokens - 1, cache->max_pages_per_req);
  const hipError_t e = launch_fill(*dims, *rot, *cache, request, hist_begin, n_tokens, k_tokens,
                                   v_tokens, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fill launch");
  return OSCAR_OK;
}

int oscar_kv_read_history(const oscar_dims* dims, const oscar_cache* cache, int32_t request, int32_t hist_begin,
                          int32_t n_tokens, float* k_out, float* v_out, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_cache(cache, true))) return rc;
  if (request < 0 || request >= cache->batch)
    return fail(OSCAR_EINVAL, "request %d outside batch %d", request, cache->batch);
  if (hist_begin < 0 || n_tokens < 0)
    return fail(OSCAR_EINVAL, "hist_begin %d / n_tokens %d must be >= 0", hist_begin, n_tokens);
  if (n_tokens == 0) return OSCAR_OK;
  if (k_out == nullptr || v_out == nullptr) return fail(OSCAR_EINVAL, "output pointers are NULL");
  const int64_t last_page = (static_cast<int64_t>(hist_begin) + n_tokens - 1) / kPage;
  if (last_page >= cache->max_pages_per_req)
    return fail(OSCAR_EINVAL, "history index %lld beyond max_pages_per_req %d",
                static_cast<long long>(hist_begin) + n_tokens - 1, cache->max_pages_per_req);
  const hipError_t e = launch_read_history(*dims, *cache, request, hist_begin, n_tokens, k_out, v_out,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read-history launch");
  return OSCAR_OK;
}

int32_t oscar_history_splits_ex(const oscar_dims* dims, int32_t batch, int32_t max_seq_len,
                                const oscar_decode_options* options) {
  g_error.clear();
  CallOpts c;
  if (check_dims(dims) || resolve_opts(*dims, options, true, false, &c)) return -1;
  if (batch < 0 || max_seq_len < 0) return -1;
  return workspace_layout(*dims, batch, max_seq_len, c.target_wg).slots;
}

int32_t oscar_history_splits(const oscar_dims* dims, int32_t batch, int32_t max_seq_len) {
  return oscar_history_splits_ex(dims, batch, max_seq_len, nullptr);
}

size_t oscar_decode_workspace_bytes(const oscar_dims* dims, int32_t batch, int32_t max_seq_len) {
  if (check_dims(dims) || batch < 0 || max_seq_len < 0) return 0;
  // the layout holds kMaxTargetWg / Hkv + B splits whatever the target
  return workspace_layout(*dims, batch, max_seq_len, kMaxTargetWg).total;
}

namespace {

// Shared body of oscar_decode_attn (out == NULL: partials only) and
// oscar_decode (merged output).
int decode_impl(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                const uint16_t* q, int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                float* out, float* lse_out, bool demote, const uint16_t* k_new, const uint16_t* v_new,
                const oscar_decode_options* options, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_rot(rot)) || (rc = check_cache(cache, true))) return rc;
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(OSCAR_EINVAL, "k_new and v_new must both be set or both be NULL");
  if (max_seq_len < 1) return fail(OSCAR_EINVAL, "max_seq_len %d < 1", max_seq_len);
  CallOpts opt;
  if ((rc = resolve_opts(*dims, options, false, false, &opt))) return rc;
  if (cache->batch == 0) return OSCAR_OK;
  if (q == nullptr || workspace == nullptr) return fail(OSCAR_EINVAL, "q or workspace is NULL");
  if (pages_for(max_seq_len) > cache->max_pages_per_req)
    return fail(OSCAR_EINVAL, "max_seq_len %d needs %d pages > max_pages_per_req %d", max_seq_len,
                pages_for(max_seq_len), cache->max_pages_per_req);
  // sizes and offsets do not depend on the target
  const size_t need = workspace_layout(*dims, cache->batch, max_seq_len, kMaxTargetWg).total;
  if (workspace_bytes < need)
    return fail(OSCAR_EINVAL, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(OSCAR_EINVAL, "workspace not 256-byte aligned");
  if ((rc = resolve_target(*dims, false, &opt))) return rc;
  const WsLayout lay = workspace_layout(*dims, cache->batch, max_seq_len, opt.target_wg);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool mfma = use_mfma(*dims, opt);
  DecodeArgs a{dims, rot, cache, q, static_cast<uint8_t*>(workspace), lay};
  history_launch_slots(lay, cache->batch, max_seq_len, &a.hist_slots, &a.sched_target);
  DemoteStep dm;
  if (demote) {
    dm = make_demote_step(*dims, *rot, *cache, k_new, v_new);
    a.demote = &dm;
  }
  hipError_t e = launch_qrot(a, s);
  if (e != hipSuccess) return hip_fail(e, "query rotation launch");
  a.ev_start = opt.ev_start;
  a.ev_stop = opt.ev_stop;
  a.clock_trace = opt.clock_trace;
  // the matrix-core launch also runs the bf16 sink/recent chunks
  e = mfma ? launch_hist_mfma(a, s) : launch_hist_valu(a, s);
  if (e != hipSuccess) return hip_fail(e, "history launch");
  if (!mfma) {
    e = launch_bf16(a, s);
    if (e != hipSuccess) return hip_fail(e, "bf16 launch");
  }
  if (out != nullptr) {
    e = launch_merge(*dims, *rot, cache->batch, a.ws, lay, out, lse_out, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return OSCAR_OK;
}

}  // namespace

int oscar_decode_attn_ex(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                         const uint16_t* q, int32_t max_seq_len, void* workspace,
                         size_t workspace_bytes, const oscar_decode_options* options, void* stream) {
  return decode_impl(dims, rot, cache, q, max_seq_len, workspace, workspace_bytes, nullptr, nullptr, false,
                     nullptr, nullptr, options, stream);
}

int oscar_decode_attn(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                      const uint16_t* q, int32_t max_seq_len, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return oscar_decode_attn_ex(dims, rot, cache, q, max_seq_len, workspace, workspace_bytes, nullptr, stream);
}

int oscar_decode_ex(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                    const uint16_t* q, int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                    float* out, float* lse_out, const oscar_decode_options* options, void* stream) {
  if (out == nullptr && cache != nullptr && cache->batch > 0) {
    g_error.clear();
    return fail(OSCAR_EINVAL, "out is NULL");
  }
  return decode_impl(dims, rot, cache, q, max_seq_len, workspace, workspace_bytes, out, lse_out, false,
                     nullptr, nullptr, options, stream);
}

int oscar_decode(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                 const uint16_t* q, int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                 float* out, float* lse_out, void* stream) {
  return oscar_decode_ex(dims, rot, cache, q, max_seq_len, workspace, workspace_bytes, out, lse_out, nullptr,
                         stream);
}

int oscar_decode_step_ex(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                         const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                         int32_t max_seq_len, void* workspace, size_t workspace_bytes, float* out,
                         float* lse_out, const oscar_decode_options* options, void* stream) {
  if (out == nullptr && cache != nullptr && cache->batch > 0) {
    g_error.clear();
    return fail(OSCAR_EINVAL, "out is NULL");
  }
  return decode_impl(dims, rot, cache, q, max_seq_len, workspace, workspace_bytes, out, lse_out, true,
                     k_new, v_new, options, stream);
}

int oscar_decode_step(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                      const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                      int32_t max_seq_len, void* workspace, size_t workspace_bytes, float* out,
                      float* lse_out, void* stream) {
  return oscar_decode_step_ex(dims, rot, cache, k_new, v_new, q, max_seq_len, workspace, workspace_bytes, out,
                              lse_out, nullptr, stream);
}

int oscar_decode_step_noalloc(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                              const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                              int32_t max_seq_len, float* out, float* lse_out, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_cache(cache, true))) return rc;
  if (max_seq_len < 1) return fail(OSCAR_EINVAL, "max_seq_len %d < 1", max_seq_len);
  if (cache->batch == 0) return OSCAR_OK;
  const size_t need = workspace_layout(*dims, cache->batch, max_seq_len, kMaxTargetWg).total;
  if (need > static_cast<size_t>(OSCAR_NOALLOC_SCRATCH_BYTES))
    return fail(OSCAR_EINVAL,
                "batch %d with %d query heads needs %zu bytes of workspace, more than the %zu-byte "
                "no-allocation scratch; use oscar_decode_step with a caller workspace",
                cache->batch, dims->num_q_heads, need, static_cast<size_t>(OSCAR_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return oscar_decode_step(dims, rot, cache, k_new, v_new, q, max_seq_len, ws, OSCAR_NOALLOC_SCRATCH_BYTES, out,
                           lse_out, stream);
}

int oscar_merge_lse(const oscar_dims* dims, const oscar_rotation* rot, int32_t batch,
                    int32_t max_seq_len, const void* workspace, size_t workspace_bytes, float* out,
                    float* lse_out, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_rot(rot))) return rc;
  if (batch < 0 || max_seq_len < 1) return fail(OSCAR_EINVAL, "batch %d / max_seq_len %d invalid", batch, max_seq_len);
  if (batch == 0) return OSCAR_OK;
  if (workspace == nullptr || out == nullptr) return fail(OSCAR_EINVAL, "workspace or out is NULL");
  // the merge reads the schedule the decode call wrote; its offsets do not
  // depend on the target
  const WsLayout lay = workspace_layout(*dims, batch, max_seq_len, kMaxTargetWg);
  if (workspace_bytes < lay.total)
    return fail(OSCAR_EINVAL, "workspace %zu bytes < %zu required", workspace_bytes, lay.total);
  const hipError_t e = launch_merge(*dims, *rot, batch, static_cast<const uint8_t*>(workspace), lay,
                                    out, lse_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return OSCAR_OK;
}

int oscar_read_history_schedule(const oscar_dims* dims, int32_t batch, const void* workspace,
                                size_t workspace_bytes, int32_t* splits, int32_t* requests,
                                int32_t capacity, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims))) return -rc;
  if (batch < 1) return -fail(OSCAR_EINVAL, "batch %d < 1", batch);
  if (workspace == nullptr || splits == nullptr || requests == nullptr)
    return -fail(OSCAR_EINVAL, "workspace, splits or requests is NULL");
  const WsLayout lay = workspace_layout(*dims, batch, 1, kMaxTargetWg);
  if (workspace_bytes < lay.total)
    return -fail(OSCAR_EINVAL, "workspace %zu bytes < %zu required", workspace_bytes, lay.total);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* ws = static_cast<const uint8_t*>(workspace);
  int32_t n = 0;
  hipError_t e = hipMemcpyAsync(&n, ws + lay.off_sched, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return -hip_fail(e, "schedule read");
  if (n < 0 || n > capacity) return -fail(OSCAR_EINVAL, "%d splits do not fit capacity %d", n, capacity);
  if (n > 0)
    e = hipMemcpyAsync(splits, ws + lay.off_sched + sizeof(int32_t), 3 * sizeof(int32_t) * n,
                       hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(requests, ws + lay.off_req, 2 * sizeof(int32_t) * batch, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return -hip_fail(e, "schedule read");
  return n;
}

size_t oscar_bf16_block_bytes(void) { return 2u * kPage * kDim * sizeof(uint16_t); }

int oscar_bf16_fill(const oscar_dims* dims, const oscar_bf16_cache* cache, int32_t request,
                    int32_t pos_begin, int32_t n_tokens, const uint16_t* k_tokens,
                    const uint16_t* v_tokens, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_bf16_cache(cache))) return rc;
  if (request < 0 || request >= cache->batch)
    return fail(OSCAR_EINVAL, "request %d outside batch %d", request, cache->batch);
  if (pos_begin < 0 || n_tokens < 0) return fail(OSCAR_EINVAL, "pos_begin %d / n_tokens %d must be >= 0", pos_begin, n_tokens);
  if (n_tokens == 0) return OSCAR_OK;
  if (k_tokens == nullptr || v_tokens == nullptr) return fail(OSCAR_EINVAL, "token pointers are NULL");
  const int64_t last_page = (static_cast<int64_t>(pos_begin) + n_tokens - 1) / kPage;
  if (last_page >= cache->max_pages_per_req)
    return fail(OSCAR_EINVAL, "position %lld beyond max_pages_per_req %d",
                static_cast<long long>(pos_begin) + n_tokens - 1, cache->max_pages_per_req);
  const hipError_t e = launch_base_fill(*dims, *cache, request, pos_begin, n_tokens, k_tokens, v_tokens,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bf16 fill launch");
  return OSCAR_OK;
}

int oscar_bf16_append(const oscar_dims* dims, const oscar_bf16_cache* cache, const uint16_t* k_new,
                      const uint16_t* v_new, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_bf16_cache(cache))) return rc;
  if (cache->batch == 0) return OSCAR_OK;
  if (k_new == nullptr || v_new == nullptr) return fail(OSCAR_EINVAL, "k_new or v_new is NULL");
  const hipError_t e = launch_base_append(*dims, *cache, k_new, v_new, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bf16 append launch");
  return OSCAR_OK;
}

size_t oscar_bf16_decode_workspace_bytes(const oscar_dims* dims, int32_t batch) {
  if (check_dims(dims) || batch < 0) return 0;
  return base_layout(*dims, batch, kMaxTargetWg).total;
}

int oscar_bf16_decode_ex(const oscar_dims* dims, const oscar_bf16_cache* cache, const uint16_t* q,
                         int32_t max_seq_len, void* workspace, size_t workspace_bytes, float* out,
                         float* lse_out, const oscar_decode_options* options, void* stream) {
  g_error.clear();
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_bf16_cache(cache))) return rc;
  if (max_seq_len < 1) return fail(OSCAR_EINVAL, "max_seq_len %d < 1", max_seq_len);
  CallOpts opt;
  if ((rc = resolve_opts(*dims, options, true, true, &opt))) return rc;
  if (cache->batch == 0) return OSCAR_OK;
  if (q == nullptr || workspace == nullptr || out == nullptr) return fail(OSCAR_EINVAL, "q, workspace or out is NULL");
  if ((max_seq_len + kPage - 1) / kPage > cache->max_pages_per_req)
    return fail(OSCAR_EINVAL, "max_seq_len %d needs %d pages > max_pages_per_req %d", max_seq_len,
                (max_seq_len + kPage - 1) / kPage, cache->max_pages_per_req);
  const BaseLayout lay = base_layout(*dims, cache->batch, opt.target_wg);
  if (workspace_bytes < lay.total)
    return fail(OSCAR_EINVAL, "workspace %zu bytes < %zu required", workspace_bytes, lay.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(OSCAR_EINVAL, "workspace not 256-byte aligned");
  const hipError_t e = launch_base_decode(*dims, *cache, q, static_cast<uint8_t*>(workspace), lay, out, lse_out,
                                          static_cast<hipStream_t>(stream), opt.ev_start, opt.ev_stop);
  if (e != hipSuccess) return hip_fail(e, "bf16 decode launch");
  return OSCAR_OK;
}

int oscar_bf16_decode(const oscar_dims* dims, const oscar_bf16_cache* cache, const uint16_t* q,
                      int32_t max_seq_len, void* workspace, size_t workspace_bytes, float* out,
                      float* lse_out, void* stream) {
  return oscar_bf16_decode_ex(dims, cache, q, max_seq_len, workspace, workspace_bytes, out, lse_out, nullptr,
                              stream);
}

}  // extern "C"
