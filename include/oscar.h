/*
 * oscar.h - C ABI of the OSCAR INT2 KV-cache decode path on MI355X (gfx950).
 *
 * OSCAR keeps each request's KV cache in three regions (page "Together AI
 * 开源 OSCAR：一种面向长上下文 LLM 服务的注意力感知 2 位 KV 缓存量化系统",
 * section "服务系统：混合精度缓存布局"; page "超越TurboQuant：Together AI把
 * 2-bit KV Cache推向真实服务", section "OSCAR的另一个关键点是"):
 *   - sink:    the first 64 tokens, bf16, unrotated;
 *   - history: every token between, stored rotated (key as k.R_K, value as
 *              v.R_V), clipped and quantized to 2-bit codes with a bf16 scale
 *              and zero point per group of G channels, 4 codes per byte;
 *   - recent:  the last 256 tokens, bf16, unrotated.
 * A decode step appends the new token to the recent window, demotes the
 * oldest recent token into history, runs attention over history and over
 * the bf16 regions separately, and merges the partial results with an
 * online-softmax (log-sum-exp) merge (same section of the second page).
 *
 * Conventions common to every call:
 *   - head_dim is 128; rotations are row-vector maps: stored = x . R, with
 *     R row-major [128][128] in float32.
 *   - "device" pointers are HIP device memory owned by the caller; the
 *     library never allocates, frees or keeps pointers after a call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns without synchronising; buffers must
 *     stay valid until that work completes.  Calls on one stream run in
 *     order; calls that touch the same cache on different streams race.
 *   - Return value: OSCAR_OK, or an error code with a message available
 *     from oscar_last_error() (thread-local).  Arguments are checked on the
 *     host before anything is enqueued; an error leaves device memory
 *     untouched.  Device-resident values (seq_lens, page_table) are trusted:
 *     the caller keeps them within the documented ranges.
 *   - No C++ exception crosses this interface.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSCAR_OK 0
#define OSCAR_EINVAL 1        /* null/inconsistent argument, workspace too small */
#define OSCAR_EUNSUPPORTED 2  /* a shape this build does not implement */
#define OSCAR_EHIP 3          /* a HIP runtime call or kernel launch failed */

/* History codebooks (oscar_dims.codebook).  Both store a 2-bit code per
 * element and a bf16 (scale, zero) pair per group of group_size channels of
 * one token; a value decodes to zero + scale * level[code].
 *   UNIFORM    levels 0, 1, 2, 3; zero = group minimum, scale = (max-min)/3,
 *              code = clamp(rint((y - zero) / scale), 0, 3) (first page,
 *              section "为什么 INT2 KV 缓存量化很难？"; second page, section
 *              "OSCAR的另一个关键点是").
 *   LLOYD_MAX  the 4-level Lloyd-Max levels of the standard normal
 *              distribution (oscar_codebook); zero = group mean, scale =
 *              population standard deviation (both in float64, then rounded
 *              to float32 and to bf16); code = the number of decision
 *              thresholds below (y - zero) / scale in float32.  The second
 *              page (its comparison with TurboQuant) says OSCAR's code pairs
 *              the rotation with a Lloyd-Max codebook; this normalisation is
 *              this library's reading of it. */
#define OSCAR_CODEBOOK_UNIFORM 0
#define OSCAR_CODEBOOK_LLOYD_MAX 1

/* Model and cache geometry.  Supported: head_dim 128, page_size 64,
 * sink_len 64, recent_len 256, group_size in {32, 64, 128},
 * num_q_heads a multiple of num_kv_heads with 1 <= Hq/Hkv <= 8, codebook
 * OSCAR_CODEBOOK_UNIFORM or OSCAR_CODEBOOK_LLOYD_MAX (zero-initialise the
 * struct: 0 is the uniform codebook).  The codebook is part of the cache
 * encoding: demote and decode one cache with the same value. */
typedef struct oscar_dims {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t group_size;
  int32_t page_size;
  int32_t sink_len;
  int32_t recent_len;
  int32_t codebook;
} oscar_dims;

/* The levels (ascending, host float32 [4]) and decision thresholds (host
 * float32 [3]) of a codebook.  For LLOYD_MAX the levels are the fixed point
 * of Lloyd's conditions for N(0, 1) (each level the mean of its cell, each
 * threshold the midpoint of its two levels), computed in float64 and rounded
 * to float32; for UNIFORM they are 0..3 and 0.5, 1.5, 2.5 (the uniform
 * quantizer rounds ties to even instead).  Host only; either pointer may be
 * NULL.  Returns OSCAR_EUNSUPPORTED for an unknown codebook. */
int oscar_codebook(int32_t codebook, float* levels, float* thresholds);

/* Fixed per-layer rotations and clip thresholds, built offline from the
 * query covariance and the score-weighted value covariance
 * (R = U . Hadamard . bit-reversal; first page, section "OSCAR 的不同之处").
 * All device, float32, read only. */
typedef struct oscar_rotation {
  const float* r_k;     /* [Hkv][128][128] */
  const float* r_v;     /* [Hkv][128][128] */
  const float* clip_k;  /* [Hkv][128], thresholds in the rotated domain, > 0 */
  const float* clip_v;  /* [Hkv][128] */
} oscar_rotation;

/* One layer's cache for a batch of requests (all device memory).
 *
 * pages:       [n_pages][Hkv][oscar_block_bytes(G)] bytes.  One block holds
 *              64 history slots of one KV head, keys and values, laid out as:
 *                bytes [0, 2048): key words; word d*64 + qk(t) holds the 2-bit
 *                  codes of channels 16d..16d+15 of slot t (d = 0..7);
 *                bytes [2048, 4096): value words; word
 *                  (c/64)*256 + ((w*16 + c%16)*4 + (c/16)%4) holds the codes
 *                  of slots 16w..16w+15 of channel c (w = 0..3);
 *                then key scale/zero, then value scale/zero: entry qk(t) is
 *                  128/G pairs {scale, zero} of bf16.
 *              Words are 32-bit little endian; element i of a word sits at
 *              bits 2i..2i+1, and the element in the top two bits of each
 *              byte (i % 4 == 3) is stored XOR 2 (a stored word is the plain
 *              packing XOR 0x80808080).  qk(t) = 16*(t/16) + 4*(t%4) + (t/4)%4.
 *              The stored channel index is the rotated one (after . R).
 * sink_k/v:    bf16 [B][Hkv][64][128]; position p < 64 at slot p.
 * recent_k/v:  bf16 [B][Hkv][256][128]; position p >= 64 at slot (p-64) % 256.
 * page_table:  int32 [B][max_pages_per_req]; history index j = p - 64 of
 *              request b lives in page page_table[b][j/64], slot j % 64.
 * seq_lens:    int32 [B]; L_b = tokens held by request b, including the
 *              current one (1 <= L_b <= max_seq_len of the call).
 * Request b holds min(L_b,64) sink, max(0,L_b-320) history and
 * min(max(L_b-64,0),256) recent tokens. */
typedef struct oscar_cache {
  uint8_t* pages;
  int64_t n_pages;
  uint16_t* sink_k;
  uint16_t* sink_v;
  uint16_t* recent_k;
  uint16_t* recent_v;
  const int32_t* page_table;
  int32_t max_pages_per_req;
  const int32_t* seq_lens;
  int32_t batch;
} oscar_cache;

/* Bytes of one (page, KV head) block for group size G: 4096 + 512*(128/G);
 * 0 for an unsupported G. */
size_t oscar_block_bytes(int32_t group_size);

/* Append + demote, one decode step (second page, section
 * "OSCAR的另一个关键点是": the oldest recent token is rotated, clipped,
 * quantized and packed into history).  seq_lens already count the new token.
 * For each request with L > 320 and each KV head, the token at position
 * L-257 is read from its recent slot, stored as y = x . R (exact products,
 * float64 accumulation, rounded once to float32), clipped
 * to [-c, c] per channel, quantized per group of G channels (zero = bf16(min),
 * scale = bf16((max-min)/3), code = clamp(rint((y-zero)/scale), 0, 3), code 0
 * when scale = 0) and packed into history index L-321 (key and value).
 * Then the new token k_new/v_new (bf16 [B][Hkv][128]) is written to its sink
 * or recent slot, which for L > 320 is the slot just freed.  k_new and v_new
 * may both be NULL (demote only).  The page holding index L-321 must be
 * allocated in page_table and owned by this request alone.  Only that slot's
 * bits change: its key words and scale/zero entries are stored whole, and
 * its two bits in each value word are cleared and set with device atomics,
 * so the page's other slots keep whatever they hold. */
int oscar_kv_demote(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                    const uint16_t* k_new, const uint16_t* v_new, void* stream);

/* Bulk form of the demotion for filling history in one launch (a prefill
 * of a long prompt): quantize n_tokens bf16 tokens k_tokens/v_tokens
 * [n_tokens][Hkv][128] (device) into history indices hist_begin ..
 * hist_begin+n_tokens-1 of request `request`, with exactly the per-token
 * arithmetic of oscar_kv_demote.  Other slots of the touched pages keep
 * their contents. */
int oscar_kv_fill_history(const oscar_dims* dims, const oscar_rotation* rot,
                          const oscar_cache* cache, int32_t request, int32_t hist_begin,
                          int32_t n_tokens, const uint16_t* k_tokens,
                          const uint16_t* v_tokens, void* stream);

/* Read history back: the dequantized stored (rotated-domain) values of
 * history indices hist_begin .. hist_begin+n_tokens-1 of request `request`,
 * zero + scale * level[code] per element, into k_out and v_out (device
 * float32 [n_tokens][Hkv][128]).  Uniform codebook: code * scale + zero with
 * one float32 rounding; Lloyd-Max: the float64 value rounded once to
 * float32.  For inspection, tests and quality metrics (the decode path never
 * forms these values).  Asynchronous on `stream`; OSCAR_EINVAL for indices
 * outside the request's page table. */
int oscar_kv_read_history(const oscar_dims* dims, const oscar_cache* cache, int32_t request,
                          int32_t hist_begin, int32_t n_tokens, float* k_out, float* v_out, void* stream);

/* Per-call choices of the decode calls (the *_ex entry points; a NULL
 * pointer, and the entry points without _ex, take every default).  The
 * library keeps no setting between calls: two threads passing different
 * options each get their own kernel and schedule.
 *   history_kernel  0 = default (the matrix-core kernel), 1 = vector-ALU
 *                   kernel, 2 = matrix-core (MFMA) kernel; both cover every
 *                   supported dims.
 *   history_target  history workgroups the split schedule aims for
 *                   (oscar_history_splits); 0 = default: the workgroups the
 *                   history kernel for these dims keeps resident on the
 *                   current device (4 SIMDs per compute unit x waves per
 *                   SIMD / waves per workgroup), at most 8192.
 *   history_start_event, history_stop_event
 *                   hipEvent_t or NULL: when both are set, the history
 *                   launch is made with hipExtLaunchKernelGGL with these as
 *                   its start and stop events, so their elapsed time is that
 *                   kernel's execution (a timing hook).
 *   history_clock_trace
 *                   device uint64 [4] or NULL: when set, the history
 *                   kernel's first workgroup writes the shader-clock cycle
 *                   counter and the constant-rate counter (the device's
 *                   hipDeviceAttributeWallClockRate, in kHz) at its start
 *                   ([0], [1]) and at its end ([2], [3]), so
 *                   ([2] - [0]) / ([3] - [1]) * wall rate is the average
 *                   shader clock over that workgroup's split (a timing
 *                   hook; the split spans most of the launch). */
typedef struct oscar_decode_options {
  int32_t history_kernel;
  int32_t history_target;
  void* history_start_event;
  void* history_stop_event;
  uint64_t* history_clock_trace;
} oscar_decode_options;

/* Upper bound on the history splits per KV head that oscar_decode_attn
 * schedules for a batch of this size.  The splits themselves are chosen on
 * the device from the lengths: with T = ceil(W / Hkv) and W the options'
 * history_target (by default the history kernel's resident workgroups on
 * the current device; on a 256-CU MI355X 3072 at G = 128 with the uniform
 * codebook and 2048 otherwise, halved for groups of more than four query
 * heads, which take two-wave workgroups), the pages per split q
 * is the smallest q >= max(4, ceil(longest / 251)) for which the batch
 * needs at most T splits, request b taking ceil(pages_b / q) splits of
 * equal size (the last one shorter); if one split per request already
 * exceeds T, q is the longest request's page count.  The bound returned is
 * T + B; -1 for invalid arguments, or when the default target is asked for
 * and no HIP device is present.  max_seq_len is not used. */
int32_t oscar_history_splits(const oscar_dims* dims, int32_t batch, int32_t max_seq_len);
int32_t oscar_history_splits_ex(const oscar_dims* dims, int32_t batch, int32_t max_seq_len,
                                const oscar_decode_options* options);

/* Workspace bytes oscar_decode_attn / oscar_merge_lse need (device memory,
 * 256-byte aligned, owned by the caller; no initialisation required). */
size_t oscar_decode_workspace_bytes(const oscar_dims* dims, int32_t batch, int32_t max_seq_len);

/* Decode attention over the three regions (second page, section
 * "OSCAR的另一个关键点是": an INT2 kernel for history with unpacking and
 * scale/zero dequantization, a bf16 kernel for sink and recent).
 * q: bf16 [B][Hq][128] (unrotated).  Query head h reads KV head h/(Hq/Hkv).
 * The query is rotated by R_K once per (request, head) (third page, method
 * paragraphs: the online overhead lives inside the decode kernels); the
 * history pages of the batch are split into page ranges on the device (see
 * oscar_history_splits) and each produces a partial output (in the rotated
 * value domain) and its log-sum-exp; the sink and recent tokens produce
 * five more partials with the unrotated query.
 * Scores use scale 1/sqrt(128).  Results go to `workspace` for
 * oscar_merge_lse.  max_seq_len >= every L_b. */
int oscar_decode_attn(const oscar_dims* dims, const oscar_rotation* rot,
                      const oscar_cache* cache, const uint16_t* q, int32_t max_seq_len,
                      void* workspace, size_t workspace_bytes, void* stream);
int oscar_decode_attn_ex(const oscar_dims* dims, const oscar_rotation* rot,
                         const oscar_cache* cache, const uint16_t* q, int32_t max_seq_len,
                         void* workspace, size_t workspace_bytes,
                         const oscar_decode_options* options, void* stream);

/* Decode attention with the merge in one call: oscar_decode_attn followed
 * by oscar_merge_lse on the same stream (out float32 [B][Hq][128], lse_out
 * float32 [B][Hq] or NULL); out may be NULL only for an empty batch. */
int oscar_decode(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                 const uint16_t* q, int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                 float* out, float* lse_out, void* stream);
int oscar_decode_ex(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                    const uint16_t* q, int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                    float* out, float* lse_out, const oscar_decode_options* options, void* stream);

/* One whole decode step: oscar_kv_demote(k_new, v_new) then
 * oscar_decode, in three launches instead of four (the demotion runs in the
 * query-rotation launch; it writes only the history slot of position L-257
 * and the new token's slot, which that launch does not read).  Same
 * arguments, requirements and results as those two calls in order. */
int oscar_decode_step(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                      const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                      int32_t max_seq_len, void* workspace, size_t workspace_bytes, float* out,
                      float* lse_out, void* stream);
int oscar_decode_step_ex(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                         const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                         int32_t max_seq_len, void* workspace, size_t workspace_bytes, float* out,
                         float* lse_out, const oscar_decode_options* options, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the same step
 * as oscar_decode_step, with its workspace taken from a device array inside
 * the library instead of a caller buffer.  The array holds
 * OSCAR_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU; each GPU the library runs
 * on keeps its copy until the process ends, and its address is looked up
 * once per device, on the first call with that device current (`stream`
 * must belong to the current device).  A batch whose workspace
 * (oscar_decode_workspace_bytes) exceeds the array is rejected with
 * OSCAR_EINVAL before anything is enqueued; with 8 KV heads that allows up
 * to 111 requests of 64 query heads or 273 of 32.  Nothing is allocated or freed: no hipMalloc, hipFree or
 * allocating library call.  The caller still owns the inputs and outputs.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams or threads with the same device) race and must be
 * ordered by the caller.  The array keeps the last call's contents; nothing
 * in it needs to start at zero.  Default options (oscar_decode_options). */
#define OSCAR_NOALLOC_SCRATCH_BYTES (64u << 20)
int oscar_decode_step_noalloc(const oscar_dims* dims, const oscar_rotation* rot, const oscar_cache* cache,
                              const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                              int32_t max_seq_len, float* out, float* lse_out, void* stream);

/* Log-sum-exp merge (second page, section "OSCAR的另一个关键点是": the
 * INT2 history and the bf16 sink/recent results are combined by an
 * online-softmax merge; first page, section "OSCAR 的不同之处": values are
 * stored as v . R_V, so the history output is rotated back by R_V^T).
 * With M the largest partial log-sum-exp, the merged output is
 * sum_i e^(lse_i - M) O_i / sum_i e^(lse_i - M) and its log-sum-exp
 * M + ln sum_i e^(lse_i - M); empty partials (lse = -inf) are skipped.  The
 * history splits are merged first, in the rotated value domain, then
 * multiplied by R_V^T and merged with the five sink/recent partials.
 * Writes out: float32 [B][Hq][128].  lse_out (may be NULL): float32 [B][Hq],
 * the natural-log log-sum-exp of all scores.  batch and max_seq_len must
 * equal those given to oscar_decode_attn for this workspace; the workspace
 * is only read. */
int oscar_merge_lse(const oscar_dims* dims, const oscar_rotation* rot, int32_t batch,
                    int32_t max_seq_len, const void* workspace, size_t workspace_bytes,
                    float* out, float* lse_out, void* stream);

/* Largest calibration sequence oscar_calibrate accepts (tokens). */
int32_t oscar_calibrate_max_tokens(void);

/* Device workspace bytes oscar_calibrate needs for n_tokens tokens; 0 on
 * invalid arguments. */
size_t oscar_calibrate_workspace_bytes(const oscar_dims* dims, int32_t n_tokens);

/* Offline calibration of one layer (first page, section "OSCAR 的不同之处";
 * second page, section "OSCAR把旋转对准attention"; third page, method
 * paragraphs).  Input: a calibration sequence of n_tokens positions,
 * device float32 q [N][Hq][128], k and v [N][Hkv][128].  For each KV head j
 * with query group G_j = {h : h / (Hq/Hkv) == j}:
 *   C_Q = mean over n and h in G_j of q_{n,h}^T q_{n,h};
 *   C_S = mean over n and h in G_j of o_{n,h}^T o_{n,h}, o_{n,h} = sum_{t<=n}
 *         softmax_t(q_{n,h} . k_t / sqrt(128)) v_t (= V^T S^T S V / N with
 *         causal attention probabilities S);
 *   R_K = U_Q . H . P_br, R_V = U_S . H . P_br, U the eigenvectors of C in
 *         descending eigenvalue order, each signed so that its entry of
 *         largest magnitude (lowest index on ties) is positive; H the
 *         normalised Sylvester Hadamard matrix; (x . P_br)_k = x_bitrev7(k);
 *   clip_K[c] = clip_percentile-th percentile (linear interpolation) of
 *         |k_n . R_K[:, c]| over n, likewise clip_V with v and R_V.
 * Statistics are float64.  Outputs: r_k, r_v device float32 [Hkv][128][128];
 * clip_k, clip_v device float32 [Hkv][128]; r_k_host, r_v_host (optional,
 * may be NULL) host float64 [Hkv][128][128].  2 <= n_tokens <=
 * oscar_calibrate_max_tokens(); 0 < clip_percentile <= 100.  This call is
 * synchronous: it waits for `stream` (the eigen-decompositions run on the
 * host between kernels) and returns when every output is written. */
int oscar_calibrate(const oscar_dims* dims, int32_t n_tokens, const float* q, const float* k,
                    const float* v, double clip_percentile, float* r_k, float* r_v, float* clip_k,
                    float* clip_v, double* r_k_host, double* r_v_host, void* workspace,
                    size_t workspace_bytes, void* stream);

/* History kernel a decode call with these options launches for dims:
 * 1 = vector-ALU, 2 = matrix-core; -1 for invalid dims or options. */
int oscar_history_kernel_for(const oscar_dims* dims, const oscar_decode_options* options);

/* Copy the history-split schedule that the last oscar_decode_attn on this
 * workspace wrote (device) to the host: splits (host int32 [capacity][3])
 * gets {request, first page, end page} per split, requests (host int32
 * [batch][2]) gets {first split, split count} per request.  Synchronous on
 * `stream`.  Returns the number of splits, or minus an OSCAR_E* code
 * (-OSCAR_EINVAL when it exceeds capacity).  For inspection and tests; the decode
 * path itself never reads the schedule back. */
int oscar_read_history_schedule(const oscar_dims* dims, int32_t batch, const void* workspace,
                                size_t workspace_bytes, int32_t* splits, int32_t* requests,
                                int32_t capacity, void* stream);

/* ---- All-bf16 KV-cache baseline -----------------------------------------
 * The cache the pages compare OSCAR against (first page, section "结果";
 * second page, section "OSCAR的另一个关键点是"): every token of a request in
 * bf16, unrotated.  Page block of one (page, KV head): keys [64][128] then
 * values [64][128], bf16 (oscar_bf16_block_bytes() = 32768); pages[n_pages]
 * [Hkv][block].  page_table[B][max_pages_per_req] maps position p to page
 * p/64, row p%64.  Same ownership and error conventions as the INT2 calls. */
typedef struct oscar_bf16_cache {
  uint16_t* pages;
  int64_t n_pages;
  const int32_t* page_table;
  int32_t max_pages_per_req;
  const int32_t* seq_lens;   /* device [B]: L including the current token */
  int32_t batch;
} oscar_bf16_cache;

size_t oscar_bf16_block_bytes(void);

/* Copy tokens [pos_begin, pos_begin + n_tokens) of one request (k_tokens,
 * v_tokens: device bf16 [n_tokens][Hkv][128]) into its pages. */
int oscar_bf16_fill(const oscar_dims* dims, const oscar_bf16_cache* cache, int32_t request,
                    int32_t pos_begin, int32_t n_tokens, const uint16_t* k_tokens,
                    const uint16_t* v_tokens, void* stream);

/* One step's append: token L_b - 1 of every request from k_new, v_new
 * (device bf16 [B][Hkv][128]); seq_lens already count it. */
int oscar_bf16_append(const oscar_dims* dims, const oscar_bf16_cache* cache, const uint16_t* k_new,
                      const uint16_t* v_new, void* stream);

/* Device workspace bytes of oscar_bf16_decode (256-byte aligned). */
size_t oscar_bf16_decode_workspace_bytes(const oscar_dims* dims, int32_t batch);

/* Decode attention over the bf16 cache: q bf16 [B][Hq][128] -> out float32
 * [B][Hq][128], lse_out float32 [B][Hq] (natural log) or NULL.  One softmax
 * over all L tokens with scale 1/sqrt(128).  Split-K over pages with the
 * same schedule rule as oscar_decode_attn (no tokens skipped; default
 * target 2048 workgroups, 1024 for eight-head groups), then a merge; three
 * launches.  With _ex, history_target sets the schedule's target and the
 * two events time the split-K launch; history_kernel must be 0. */
int oscar_bf16_decode(const oscar_dims* dims, const oscar_bf16_cache* cache, const uint16_t* q,
                      int32_t max_seq_len, void* workspace, size_t workspace_bytes, float* out,
                      float* lse_out, void* stream);
int oscar_bf16_decode_ex(const oscar_dims* dims, const oscar_bf16_cache* cache, const uint16_t* q,
                         int32_t max_seq_len, void* workspace, size_t workspace_bytes, float* out,
                         float* lse_out, const oscar_decode_options* options, void* stream);

/* Thread-local text of the last error ("" if none). */
const char* oscar_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
