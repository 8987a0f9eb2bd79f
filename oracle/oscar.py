"""Plain CPU oracle of OSCAR's INT2 KV-cache decode path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  The product
path (the HIP library and its binding) never imports or calls it, and this
module imports nothing from the product.

Everything here is slow and direct: float64 numpy, with a library routine
(a matmul, ``eigh``, ``percentile``) standing in for a single step where the
definition allows, and no blocking, fusion or reordering beyond what each
definition states.

Sources (cited by short label below):

  [A] "Together AI 开源 OSCAR：一种面向长上下文 LLM 服务的注意力感知 2 位 KV
      缓存量化系统" (news.chathome.org)
  [B] "超越TurboQuant：Together AI把2-bit KV Cache推向真实服务" (haoling.cc)
  [C] "OSCAR: открытая система двухбитного сжатия KV-кэша" (Telegram post)

Readings taken where the pages are silent are marked READING.  They are listed
in the design notes with the alternatives that were rejected.

Parity status: every public function below is pinned by a ``-m "not gpu"``
test against something other than itself: a closed form, an invariant, a
library routine, brute force on tiny inputs, or the figures the pages print.
No function is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 128        # head dimension of every model the pages evaluate
SINK = 64             # [A] §服务系统：混合精度缓存布局; [B] §OSCAR的另一个关键点是; [C]
RECENT = 256          # same three places
PAGE = 64             # paged-KV page size of the synthetic workloads
LEVELS = 4            # INT2 has four levels: [A] §为什么 INT2 KV 缓存量化很难？
CODES_PER_BYTE = 4    # four 2-bit values per byte: [B] §OSCAR的另一个关键点是
BF16_TOKENS = SINK + RECENT


# ===========================================================================
# Offline calibration: [A] §OSCAR 的不同之处; [B] §OSCAR把旋转对准attention;
# [C] (method paragraphs: calibration set, Hadamard, bit reversal)
# ===========================================================================

def query_covariance(q: np.ndarray) -> np.ndarray:
    """Empirical query covariance C_Q = (1/N) sum_n q_n^T q_n.

    [A] §OSCAR 的不同之处 defines C_Q over calibration queries (row vectors).
    READING: for grouped-query attention the g query heads that share one KV
    head are pooled, so ``q`` is [N][g][128] and the mean runs over N*g rows.
    This is the weight that the logit-error identity puts on the shared key
    error, summed over the group; with g = 1 it is the pages' formula.
    """
    rows = np.asarray(q, dtype=np.float64).reshape(-1, HEAD_DIM)
    return rows.T @ rows / rows.shape[0]


def causal_attention_outputs(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Rows of S V for one head: S = causal softmax(q k^T / sqrt(d)).

    ``q``, ``k``, ``v`` are [N][128]; query n sees keys 0..n.
    READING: S holds post-softmax attention probabilities (the matrix that
    weights the value rows to form the attention output, [A] §OSCAR 的不同之处),
    under the causal mask of a prefill over the calibration sequence, with
    the usual 1/sqrt(d) scale.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    scores = q @ k.T / math.sqrt(HEAD_DIM)
    scores[np.triu_indices(n, 1)] = -np.inf
    scores -= scores.max(axis=1, keepdims=True)
    p = np.exp(scores)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def score_weighted_value_covariance(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V, [A] §OSCAR 的不同之处.

    ``q`` is [N][g][128]; ``k``, ``v`` are [N][128] of the shared KV head.
    (S V)^T (S V) equals V^T S^T S V.  READING: pooled over the g query
    heads of the group like :func:`query_covariance`.
    """
    q = np.asarray(q, dtype=np.float64)
    n, g = q.shape[0], q.shape[1]
    total = np.zeros((HEAD_DIM, HEAD_DIM))
    for h in range(g):
        o = causal_attention_outputs(q[:, h, :], k, v)
        total += o.T @ o
    return total / (n * g)


def eig_descending(c: np.ndarray):
    """Eigen-decomposition C = U diag(lam) U^T with eigenvalues descending.

    The eigenvectors form the rotation basis ([A] §OSCAR 的不同之处).
    ``numpy.linalg.eigh`` is the library step.  READING (sign is silent on
    the pages): each column is flipped so that its entry of largest magnitude
    is positive, the lowest index winning ties.  Descending order follows the
    "importance hierarchy" the same section describes.
    """
    lam, u = np.linalg.eigh(np.asarray(c, dtype=np.float64))
    order = np.argsort(-lam, kind="stable")
    lam, u = lam[order], u[:, order].copy()
    for j in range(u.shape[1]):
        i = int(np.argmax(np.abs(u[:, j])))
        if u[i, j] < 0:
            u[:, j] = -u[:, j]
    return lam, u


def hadamard(n: int = HEAD_DIM) -> np.ndarray:
    """Normalised Sylvester Hadamard matrix H with H[i][k] = (-1)^popcount(i&k)/sqrt(n).

    READING: the pages name only "Hadamard"; natural (Sylvester) order.
    """
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != n:
        raise ValueError("n must be a power of two")
    return h / math.sqrt(n)


def bit_reverse(i: int, bits: int = 7) -> int:
    """Reverse the lowest ``bits`` bits of i."""
    r = 0
    for b in range(bits):
        r |= ((i >> b) & 1) << (bits - 1 - b)
    return r


def bit_reversal_matrix(n: int = HEAD_DIM) -> np.ndarray:
    """Permutation P_br with P[i][bitrev(i)] = 1, so (x P)_k = x_{bitrev(k)}.

    [A] §OSCAR 的不同之处 and [B] §OSCAR把旋转对准attention: the reordering
    makes every quantization group draw channels from every level of the
    importance order.
    """
    bits = int(round(math.log2(n)))
    p = np.zeros((n, n))
    for i in range(n):
        p[i, bit_reverse(i, bits)] = 1.0
    return p


def composite_rotation(u: np.ndarray) -> np.ndarray:
    """R = U . H_Had . P_br ([A] §OSCAR 的不同之处; [B] §OSCAR把旋转对准attention)."""
    return np.asarray(u, dtype=np.float64) @ hadamard(u.shape[0]) @ bit_reversal_matrix(u.shape[0])


def clip_thresholds(x: np.ndarray, r: np.ndarray, pct: float = 99.9) -> np.ndarray:
    """Per-channel clipping thresholds in the rotated domain, float32 [128].

    The thresholds are calibrated offline with the rotation and fixed at
    inference ([B] §OSCAR把旋转对准attention; [C]).  READING: the
    ``pct``-th percentile of |x R| per channel over the calibration rows,
    with linear interpolation (numpy's default), applied symmetrically.
    """
    y = np.asarray(x, dtype=np.float64).reshape(-1, HEAD_DIM) @ r
    return np.percentile(np.abs(y), pct, axis=0).astype(np.float32)


def calibrate_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, pct: float = 99.9) -> dict:
    """Calibrate one KV head from a calibration sequence.

    ``q`` [N][g][128] are the queries of the g heads sharing this KV head,
    ``k`` and ``v`` [N][128].  Returns float64 rotations R_K = U_Q H P and
    R_V = U_S H P, the float32 clip thresholds for K and V, and the
    eigenvalues of C_Q and C_S.
    """
    lam_q, u_q = eig_descending(query_covariance(q))
    lam_s, u_s = eig_descending(score_weighted_value_covariance(q, k, v))
    r_k = composite_rotation(u_q)
    r_v = composite_rotation(u_s)
    return {
        "r_k": r_k, "r_v": r_v,
        "clip_k": clip_thresholds(k, r_k, pct), "clip_v": clip_thresholds(v, r_v, pct),
        "lam_q": lam_q, "lam_s": lam_s,
    }


def calibrate(q: np.ndarray, k: np.ndarray, v: np.ndarray, pct: float = 99.9) -> dict:
    """Calibrate every KV head ("for each layer and each head",
    [B] §OSCAR把旋转对准attention).  ``q`` [N][Hq][128], ``k``/``v`` [N][Hkv][128];
    query head h belongs to KV head h // (Hq / Hkv).  Rotations are returned
    in float64 and as the float32 copies the runtime consumes.
    """
    hq, hkv = q.shape[1], k.shape[1]
    g = hq // hkv
    heads = [calibrate_head(q[:, j * g:(j + 1) * g, :], k[:, j, :], v[:, j, :], pct)
             for j in range(hkv)]
    out = {key: np.stack([h[key] for h in heads]) for key in heads[0]}
    out["r_k32"] = out["r_k"].astype(np.float32)
    out["r_v32"] = out["r_v"].astype(np.float32)
    return out


# ===========================================================================
# Demotion: rotate -> clip -> quantize -> pack ([B] §OSCAR的另一个关键点是)
# ===========================================================================

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """Value of bfloat16 bit patterns, as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def rotate(x: np.ndarray, r32: np.ndarray) -> np.ndarray:
    """Stored-domain value y = x . R, rounded once to float32.

    ``x`` [n][128] (the bf16 token values), ``r32`` the float32 rotation.
    Products of a bf16 and a float32 are exact in float64; the sum is
    float64 and rounded once.
    """
    return (np.asarray(x, dtype=np.float64) @ np.asarray(r32, dtype=np.float64)).astype(np.float32)


def clip(y: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Clamp each channel to [-c_k, c_k] (float32)."""
    c = np.asarray(c, dtype=np.float32)
    return np.minimum(np.maximum(np.asarray(y, dtype=np.float32), -c), c)


def quantize_groups(y: np.ndarray, group: int):
    """Asymmetric 4-level quantization per token and group of ``group`` channels.

    [A] §为什么 INT2 KV 缓存量化很难？ (four levels) and
    [B] §OSCAR的另一个关键点是 (dequantization by scale and zero point).
    READING: zero point = group minimum, scale = (max - min) / 3, both held
    in bfloat16; code = clamp(rint((y - z) / s), 0, 3) with IEEE float32
    subtraction and division and ties to even; a group with s = 0 gets code 0.

    Returns codes uint8 [n][128] and scale, zero as float32 [n][128/group].
    """
    y = np.asarray(y, dtype=np.float32)
    n = y.shape[0]
    ng = HEAD_DIM // group
    yg = y.reshape(n, ng, group)
    mn = yg.min(axis=2)
    mx = yg.max(axis=2)
    s = bf16_round(((mx - mn).astype(np.float32) / np.float32(3.0)).astype(np.float32))
    z = bf16_round(mn)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = ((yg - z[:, :, None]).astype(np.float32) / s[:, :, None]).astype(np.float32)
    codes = np.clip(np.rint(t), 0, LEVELS - 1)
    codes = np.where(s[:, :, None] == 0, 0, codes)
    return codes.astype(np.uint8).reshape(n, HEAD_DIM), s, z


def dequantize(codes: np.ndarray, s: np.ndarray, z: np.ndarray, group: int) -> np.ndarray:
    """y_hat = code * s + z in float32 (code * s is exact)."""
    n = codes.shape[0]
    ng = HEAD_DIM // group
    c = codes.reshape(n, ng, group).astype(np.float32)
    out = c * s[:, :, None].astype(np.float32) + z[:, :, None].astype(np.float32)
    return out.astype(np.float32).reshape(n, HEAD_DIM)


# ---------------------------------------------------------------------------
# Lloyd-Max codebook variant.  [B] (the paragraph comparing OSCAR with
# TurboQuant) says only that OSCAR's code repository pairs the
# attention-aware rotation with a Lloyd-Max codebook.
# READING: the codebook is the 4-level Lloyd-Max (minimum mean-squared
# error) quantizer of the standard normal distribution, applied to each
# group after normalising it by its mean and standard deviation, which take
# the places of the uniform quantizer's zero point and scale: zero = mean,
# scale = population standard deviation, both computed in float64, rounded
# to float32 and then to bfloat16.  u = (y - zero) / scale in IEEE float32;
# the code is the number of float32 decision thresholds strictly below u
# (the nearest level, ties to the lower one); a group with scale 0 gets code
# 0.  The stored codebook is the float32 levels; a value decodes to
# zero + scale * level[code].  The decision thresholds are the float64
# midpoints of adjacent float64 levels, rounded to float32.
# ---------------------------------------------------------------------------

def _normal_pdf(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _normal_tail(x: float) -> float:
    """P(X > x) for X ~ N(0, 1), x >= 0 (inf gives 0)."""
    return 0.0 if x == math.inf else 0.5 * math.erfc(x / math.sqrt(2.0))


def lloyd_max_gaussian(n_levels: int = LEVELS, max_iter: int = 100000):
    """Lloyd-Max quantizer of N(0, 1) with an even number of levels.

    Lloyd's alternation on the positive half (the density is symmetric, and
    so is the optimum): the thresholds are the midpoints of adjacent levels,
    and each level is the mean of N(0, 1) restricted to its cell, which on
    (a, b) is (pdf(a) - pdf(b)) / P(a < X < b).  Starts from levels
    1/2, 3/2, ... and stops once an iteration moves no level by more than
    1e-15 (float64 resolution; about 60 iterations for four levels), then
    takes one more.  Returns float64 (levels ascending [n], thresholds [n - 1]).
    """
    if n_levels % 2 or n_levels < 2:
        raise ValueError("n_levels must be even and >= 2")
    half = n_levels // 2
    lev = [k + 0.5 for k in range(half)]
    extra = 1
    for _ in range(max_iter):
        edges = [0.0] + [(lev[k] + lev[k + 1]) / 2 for k in range(half - 1)] + [math.inf]
        new = []
        for a, b in zip(edges[:-1], edges[1:]):
            pdf_b = 0.0 if b == math.inf else _normal_pdf(b)
            new.append((_normal_pdf(a) - pdf_b) / (_normal_tail(a) - _normal_tail(b)))
        settled = max(abs(x - y) for x, y in zip(new, lev)) <= 1e-15
        lev = new
        if settled:
            if extra == 0:
                break
            extra -= 1
    levels = np.array([-x for x in reversed(lev)] + lev, dtype=np.float64)
    thresholds = (levels[:-1] + levels[1:]) / 2
    return levels, thresholds


def lloyd_max_codebook():
    """The stored codebook: float32 levels [4] and float32 thresholds [3]."""
    lev, thr = lloyd_max_gaussian(LEVELS)
    return lev.astype(np.float32), thr.astype(np.float32)


def quantize_groups_lloyd(y: np.ndarray, group: int):
    """Lloyd-Max codebook quantization per token and group (READING above).

    Returns codes uint8 [n][128] and scale (standard deviation), zero (mean)
    as float32 [n][128/group], both bfloat16 values.
    """
    y = np.asarray(y, dtype=np.float32)
    n = y.shape[0]
    ng = HEAD_DIM // group
    yg = y.reshape(n, ng, group)
    y64 = yg.astype(np.float64)
    mean = y64.sum(axis=2) / group
    var = ((y64 - mean[:, :, None]) ** 2).sum(axis=2) / group
    z = bf16_round(mean.astype(np.float32))
    s = bf16_round(np.sqrt(var).astype(np.float32))
    _, thr = lloyd_max_codebook()
    with np.errstate(divide="ignore", invalid="ignore"):
        u = ((yg - z[:, :, None]).astype(np.float32) / s[:, :, None]).astype(np.float32)
    codes = sum((u > t).astype(np.int64) for t in thr)
    codes = np.where(s[:, :, None] == 0, 0, codes)
    return codes.astype(np.uint8).reshape(n, HEAD_DIM), s, z


def dequantize_lloyd(codes: np.ndarray, s: np.ndarray, z: np.ndarray, group: int) -> np.ndarray:
    """y_hat = zero + scale * level[code] with the float32 levels, in float64."""
    lev, _ = lloyd_max_codebook()
    n = codes.shape[0]
    ng = HEAD_DIM // group
    lv = lev.astype(np.float64)[codes.reshape(n, ng, group)]
    out = z[:, :, None].astype(np.float64) + s[:, :, None].astype(np.float64) * lv
    return out.reshape(n, HEAD_DIM)


CODEBOOKS = ("uniform", "lloyd-max")


def quantize(y: np.ndarray, group: int, codebook: str = "uniform"):
    """Dispatch on the codebook: "uniform" (min/max, the pages' INT2) or
    "lloyd-max" (the variant above)."""
    if codebook == "uniform":
        return quantize_groups(y, group)
    if codebook == "lloyd-max":
        return quantize_groups_lloyd(y, group)
    raise ValueError(codebook)


def dequantize_any(codes, s, z, group: int, codebook: str = "uniform") -> np.ndarray:
    """Dequantized history in the stored domain for either codebook."""
    if codebook == "uniform":
        return dequantize(codes, s, z, group)
    if codebook == "lloyd-max":
        return dequantize_lloyd(codes, s, z, group)
    raise ValueError(codebook)


def demote(x_bits: np.ndarray, r32: np.ndarray, clip32: np.ndarray, group: int, codebook: str = "uniform"):
    """Rotate, clip and quantize bf16 tokens [n][128] (bit patterns) of one
    KV head: the per-token work of the fused demotion kernel
    ([B] §OSCAR的另一个关键点是).  Returns (codes, scale, zero)."""
    x = bf16_value(x_bits)
    return quantize(clip(rotate(x, r32), clip32), group, codebook)


# ---------------------------------------------------------------------------
# Page-block layout: the packed bytes of one (page, KV head).
#
# READING: the pages fix only "four 2-bit values per byte".  A block holds
# PAGE = 64 token slots and is laid out as follows (all words 32-bit little
# endian; inside a word, element i sits at bits 2i..2i+1, LSB first):
#   bytes [0, 2048)      K words: word d*64 + qk_order(t) holds the codes of
#                        channels 16d..16d+15 of slot t (d = 0..7)
#   bytes [2048, 4096)   V words: word (c//64)*256 + ((w*16 + c%16)*4 + (c//16)%4)
#                        holds the codes of slots 16w..16w+15 of channel c
#   then K scale/zero, then V scale/zero: entry qk_order(t) is 128/G pairs
#   (scale, zero) of bfloat16, 4*(128/G) bytes per slot.
# qk_order(t) = 16*(t//16) + 4*(t%4) + (t//4)%4.
# The code in the top two bits of every byte (element i with i % 4 == 3) is
# stored XOR 2: a stored word is the plain packing XOR 0x80808080.  (A
# storage choice with no effect on any value: that element, masked in
# place, then reads as the signed byte 64 (code - 2).)
# ---------------------------------------------------------------------------

TOP_FIELD_FLIP = 0x80808080


def qk_order(t: int) -> int:
    return 16 * (t // 16) + 4 * (t % 4) + (t // 4) % 4


def block_bytes(group: int) -> int:
    return 4096 + 2 * PAGE * (HEAD_DIM // group) * 4


def _bf16_bits_of(x: np.ndarray) -> np.ndarray:
    """Bit pattern of values that are already bfloat16-representable."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def pack_block(codes_k, s_k, z_k, codes_v, s_v, z_v, group: int) -> np.ndarray:
    """Pack 64 slots (codes uint8 [64][128], scale/zero [64][128/G]) into one block."""
    ng = HEAD_DIM // group
    words = np.zeros(1024, dtype=np.uint32)
    for t in range(PAGE):
        for d in range(8):
            w = 0
            for i in range(16):
                w |= int(codes_k[t][16 * d + i]) << (2 * i)
            words[d * 64 + qk_order(t)] = w ^ TOP_FIELD_FLIP
    for c in range(HEAD_DIM):
        for wi in range(4):
            w = 0
            for i in range(16):
                w |= int(codes_v[16 * wi + i][c]) << (2 * i)
            words[512 + (c // 64) * 256 + (wi * 16 + c % 16) * 4 + (c // 16) % 4] = w ^ TOP_FIELD_FLIP
    sz = np.zeros((2, PAGE, ng, 2), dtype=np.uint16)
    for t in range(PAGE):
        o = qk_order(t)
        sz[0, o, :, 0] = _bf16_bits_of(np.asarray(s_k[t], dtype=np.float32))
        sz[0, o, :, 1] = _bf16_bits_of(np.asarray(z_k[t], dtype=np.float32))
        sz[1, o, :, 0] = _bf16_bits_of(np.asarray(s_v[t], dtype=np.float32))
        sz[1, o, :, 1] = _bf16_bits_of(np.asarray(z_v[t], dtype=np.float32))
    out = np.concatenate([words.astype("<u4").view(np.uint8), sz.astype("<u2").reshape(-1).view(np.uint8)])
    assert out.size == block_bytes(group)
    return out


def unpack_block(block: np.ndarray, group: int):
    """Inverse of :func:`pack_block`: codes_k, s_k, z_k, codes_v, s_v, z_v."""
    ng = HEAD_DIM // group
    block = np.asarray(block, dtype=np.uint8)
    words = block[:4096].view("<u4").astype(np.int64)
    codes_k = np.zeros((PAGE, HEAD_DIM), dtype=np.uint8)
    codes_v = np.zeros((PAGE, HEAD_DIM), dtype=np.uint8)
    for t in range(PAGE):
        for d in range(8):
            w = int(words[d * 64 + qk_order(t)]) ^ TOP_FIELD_FLIP
            for i in range(16):
                codes_k[t][16 * d + i] = (w >> (2 * i)) & 3
    for c in range(HEAD_DIM):
        for wi in range(4):
            w = int(words[512 + (c // 64) * 256 + (wi * 16 + c % 16) * 4 + (c // 16) % 4]) ^ TOP_FIELD_FLIP
            for i in range(16):
                codes_v[16 * wi + i][c] = (w >> (2 * i)) & 3
    sz = block[4096:].view("<u2").reshape(2, PAGE, ng, 2)
    inv = [qk_order(t) for t in range(PAGE)]
    vals = bf16_value(sz).astype(np.float32)
    s_k = np.stack([vals[0, inv[t], :, 0] for t in range(PAGE)])
    z_k = np.stack([vals[0, inv[t], :, 1] for t in range(PAGE)])
    s_v = np.stack([vals[1, inv[t], :, 0] for t in range(PAGE)])
    z_v = np.stack([vals[1, inv[t], :, 1] for t in range(PAGE)])
    return codes_k, s_k, z_k, codes_v, s_v, z_v


# ===========================================================================
# Three-region cache and decode attention
# ([A] §服务系统：混合精度缓存布局; [B] §OSCAR的另一个关键点是; [C])
# ===========================================================================

def regions(L: int):
    """Token counts (sink, history, recent) of a request holding L tokens.

    The first 64 tokens stay bf16 (sink), the last 256 before the current
    position stay bf16 (recent) and everything between is INT2 history.
    READING: the newly appended token is part of the recent window it attends.
    """
    n_sink = min(L, SINK)
    n_hist = max(0, L - BF16_TOKENS)
    n_recent = min(max(L - SINK, 0), RECENT)
    return n_sink, n_hist, n_recent


def quantized_history(k_bits: np.ndarray, v_bits: np.ndarray, r_k32, r_v32, clip_k, clip_v,
                      group: int, codebook: str = "uniform"):
    """Demote every history token of one (request, KV head).

    ``k_bits``/``v_bits`` are the bf16 tokens at history positions
    64 .. L-257 ([n_hist][128]).  Each token is demoted on its own, so the
    result does not depend on the order in which tokens left the window.
    """
    hk = demote(k_bits, r_k32, clip_k, group, codebook)
    hv = demote(v_bits, r_v32, clip_v, group, codebook)
    return hk, hv


def attend(q_bits: np.ndarray, bf16_k: np.ndarray, bf16_v: np.ndarray,
           hist_k_hat: np.ndarray, hist_v_hat: np.ndarray,
           r_k32: np.ndarray, r_v32: np.ndarray):
    """Decode attention of the g query heads of one KV head, float64.

    ``q_bits`` [g][128] bf16 bits (unrotated); ``bf16_k``/``bf16_v`` the
    sink and recent tokens ([n][128] bf16 bits, unrotated); ``hist_*_hat``
    the dequantized history in the stored (rotated) domain, [n_h][128].

    Keys are stored as K R_K and the query is rotated by the same R_K, so
    q R_K . k_hat equals q . (k_hat R_K^T); values are stored as V R_V and the
    history part of the output is rotated back by R_V^T.  One softmax over
    all tokens, scale 1/sqrt(128), natural-log LSE.  Returns (out [g][128],
    lse [g]).
    """
    q = bf16_value(q_bits)
    kb = bf16_value(bf16_k)
    vb = bf16_value(bf16_v)
    rk = np.asarray(r_k32, dtype=np.float64)
    rv = np.asarray(r_v32, dtype=np.float64)
    kh = np.asarray(hist_k_hat, dtype=np.float64)
    vh = np.asarray(hist_v_hat, dtype=np.float64)
    scale = 1.0 / math.sqrt(HEAD_DIM)
    s_b = q @ kb.T * scale                       # [g][n_b]
    s_h = (q @ rk) @ kh.T * scale                # [g][n_h]
    m = np.max(np.concatenate([s_b, s_h], axis=1), axis=1, keepdims=True)
    p_b = np.exp(s_b - m)
    p_h = np.exp(s_h - m)
    denom = p_b.sum(axis=1) + p_h.sum(axis=1)
    o = p_b @ vb + (p_h @ vh) @ rv.T
    return o / denom[:, None], m[:, 0] + np.log(denom)


def partial_attend(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray):
    """Softmax attention of float64 queries [g][128] over one token subset,
    returning the normalised partial output and its LSE (-inf when empty)."""
    g = q_rows.shape[0]
    if k_rows.shape[0] == 0:
        return np.zeros((g, HEAD_DIM)), np.full(g, -np.inf)
    s = q_rows @ k_rows.T / math.sqrt(HEAD_DIM)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1)
    return (p @ v_rows) / l[:, None], m[:, 0] + np.log(l)


def merge_lse(outs, lses):
    """Online-softmax merge of partial results ([B] §OSCAR的另一个关键点是):
    O = sum_i e^{lse_i - M} O_i / sum_i e^{lse_i - M}, lse = M + ln sum_i e^{lse_i - M},
    skipping empty partials (lse = -inf)."""
    lses = np.stack(lses)            # [n][g]
    outs = np.stack(outs)            # [n][g][128]
    mx = np.max(lses, axis=0)
    w = np.where(np.isfinite(lses), np.exp(lses - mx[None]), 0.0)
    tot = w.sum(axis=0)
    return (w[:, :, None] * outs).sum(axis=0) / tot[:, None], mx + np.log(tot)


def bf16_cache_attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray):
    """Decode attention over an all-bf16 KV cache: the baseline the pages
    measure INT2 against ([A] §结果 and [B] §OSCAR的另一个关键点是 compare
    with a BF16 KV cache).  q_bits [g][128], k_bits and v_bits [L][128]
    bf16 bit patterns, no rotation, no quantization; one softmax with scale
    1/sqrt(128) in float64.  Returns (out [g][128], natural-log lse [g])."""
    return partial_attend(bf16_value(q_bits), bf16_value(k_bits), bf16_value(v_bits))


def bits_per_element(L: int, group: int) -> float:
    """Average stored bits per KV element of a request holding L tokens:
    16 for the 320 bf16 tokens, 2 + 2*16/G for history (bf16 scale and zero
    per group)."""
    n_bf16 = min(L, BF16_TOKENS)
    n_hist = max(0, L - BF16_TOKENS)
    return (n_bf16 * 16 + n_hist * (2 + 32 / group)) / L


def history_memory_ratio(group: int, with_metadata: bool = True) -> float:
    """Bytes of bf16 history over bytes of INT2 history."""
    return 16 / (2 + 32 / group) if with_metadata else 16 / 2


# ===========================================================================
# Whole request: the state after one decode step
# ===========================================================================

def request_attention(q_bits: np.ndarray, k_tokens: np.ndarray, v_tokens: np.ndarray,
                      r_k32: np.ndarray, r_v32: np.ndarray, clip_k: np.ndarray,
                      clip_v: np.ndarray, group: int, codebook: str = "uniform"):
    """Attention output of one request after its latest append and demotion.

    ``q_bits`` [Hq][128]; ``k_tokens``/``v_tokens`` [L][Hkv][128] bf16 bits
    of every token so far (position order); rotations [Hkv][128][128] and
    clips [Hkv][128] float32; ``codebook`` "uniform" or "lloyd-max".
    Returns out [Hq][128] float64 and lse [Hq].
    """
    L, hkv = k_tokens.shape[0], k_tokens.shape[1]
    hq = q_bits.shape[0]
    g = hq // hkv
    n_sink, n_hist, n_recent = regions(L)
    out = np.zeros((hq, HEAD_DIM))
    lse = np.zeros(hq)
    bf16_pos = list(range(n_sink)) + list(range(L - n_recent, L))
    for j in range(hkv):
        hist = slice(SINK, SINK + n_hist)
        (ck, sk, zk), (cv, sv, zv) = quantized_history(
            k_tokens[hist, j], v_tokens[hist, j], r_k32[j], r_v32[j], clip_k[j], clip_v[j], group, codebook)
        kh = dequantize_any(ck, sk, zk, group, codebook)
        vh = dequantize_any(cv, sv, zv, group, codebook)
        o, l = attend(q_bits[j * g:(j + 1) * g], k_tokens[bf16_pos, j], v_tokens[bf16_pos, j],
                      kh, vh, r_k32[j], r_v32[j])
        out[j * g:(j + 1) * g] = o
        lse[j * g:(j + 1) * g] = l
    return out, lse
