"""Seeded synthetic inputs shared by the oracle-side tests and the GPU harness.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, clipping, quantization or attention).

Generator
---------
Counter-based: the i-th 64-bit draw of stream ``key`` is the SplitMix64
output for state ``key + (i + 1) * 0x9E3779B97F4A7C15`` (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014; the
finaliser below is the published SplitMix64 mix).  Any draw can therefore be
produced independently, on the host (this file) or on the GPU
(``synth/fill.hip``, the same definition written in HIP C++).

Normal variates use the Irwin-Hall construction with twelve 16-bit uniforms
(three 64-bit draws): ``x = (sum - 12 * 32767.5) / 65536``.  Every step is
integer arithmetic followed by one exact power-of-two scaling, so host and
GPU produce bit-identical float32 values (variance 1 - 2^-32, support
+-6 sigma).  Multiplying by an outlier factor of 10 or 20 stays exact in
float32; the final bfloat16 rounding is round-to-nearest-even done on the
integer bit pattern.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_S30, _S27, _S31 = np.uint64(30), np.uint64(27), np.uint64(31)

# Stream identifiers: one per synthetic tensor family.
STREAM_K_CACHE = 1
STREAM_V_CACHE = 2
STREAM_CAL_Q = 3
STREAM_CAL_K = 4
STREAM_CAL_V = 5
STREAM_QUERY = 6
STREAM_QSIGMA = 7
STREAM_OUTLIER = 8
STREAM_PAGES = 9
STREAM_LENS = 10

POS_BITS = 21          # positions < 2^21 per (source, kv head)
KVH_SLOTS = 64         # kv heads per source slot in the cache index
SHARED_SRC = 65535     # source id for tokens of a shared prefix


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> _S30)) * _M1
        z = (z ^ (z >> _S27)) * _M2
    return z ^ (z >> _S31)


def stream_key(seed: int, stream: int) -> np.uint64:
    """64-bit key of one stream: mix(mix(seed) ^ mix(stream + golden))."""
    with np.errstate(over="ignore"):
        a = mix64(np.array([seed & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))
        b = mix64(np.array([stream], dtype=np.uint64) + GOLDEN)
        return mix64(a ^ b)[0]


def rand64(key: np.uint64, counter: np.ndarray) -> np.ndarray:
    """Draw number ``counter`` of stream ``key`` (vectorised over counter)."""
    c = np.asarray(counter, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + (c + np.uint64(1)) * GOLDEN)


def normal_f32(key: np.uint64, index: np.ndarray) -> np.ndarray:
    """Irwin-Hall(12) approximately standard normal float32 for each index:
    the twelve 16-bit fields of draws 3*index, 3*index+1, 3*index+2 summed."""
    idx = np.asarray(index, dtype=np.uint64)
    shape = idx.shape
    counters = (idx.reshape(-1, 1) * np.uint64(3) + np.arange(3, dtype=np.uint64)[None, :]).reshape(-1)
    r = np.ascontiguousarray(rand64(key, counters), dtype="<u8")
    total = r.view("<u2").reshape(-1, 12).sum(axis=1, dtype=np.int64)
    # (sum - 12 * 32767.5) * 2^-16: an integer below 2^19 times a power of two
    return ((total - 393210).astype(np.float32) * np.float32(2.0 ** -16)).reshape(shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern -> float32 value (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Model-level synthetic properties
# ---------------------------------------------------------------------------

def outlier_scales(seed: int, num_kv_heads: int, n_k: int = 4, n_v: int = 2,
                   k_factor: float = 20.0, v_factor: float = 10.0):
    """Per (kv head, channel) multipliers: ``n_k`` key channels scaled by
    ``k_factor`` and ``n_v`` value channels by ``v_factor``, chosen by a
    seeded partial Fisher-Yates shuffle of the 128 channels.

    Returns float32 arrays ``(k_scale, v_scale)`` of shape [Hkv][128].
    """
    key = stream_key(seed, STREAM_OUTLIER)
    ks = np.ones((num_kv_heads, 128), dtype=np.float32)
    vs = np.ones((num_kv_heads, 128), dtype=np.float32)
    for j in range(num_kv_heads):
        perm = list(range(128))
        draws = rand64(key, np.arange(j * 256, j * 256 + 128, dtype=np.uint64))
        for i in range(n_k + n_v):
            r = i + int(draws[i] % np.uint64(128 - i))
            perm[i], perm[r] = perm[r], perm[i]
        for c in perm[:n_k]:
            ks[j, c] = k_factor
        for c in perm[n_k:n_k + n_v]:
            vs[j, c] = v_factor
    return ks, vs


def query_sigma(seed: int, num_q_heads: int, anisotropic: bool) -> np.ndarray:
    """Per (query head, channel) standard deviation, float64 [Hq][128].

    Anisotropic: sigma = exp(z) with z ~ N(0, 1) per channel (log-normal,
    sigma parameter 1); otherwise all ones.
    """
    if not anisotropic:
        return np.ones((num_q_heads, 128), dtype=np.float64)
    key = stream_key(seed, STREAM_QSIGMA)
    z = normal_f32(key, np.arange(num_q_heads * 128, dtype=np.uint64)).astype(np.float64)
    return np.exp(z).reshape(num_q_heads, 128)


# ---------------------------------------------------------------------------
# Token streams
# ---------------------------------------------------------------------------

def cache_index(src: int, kvh: int, pos: np.ndarray, ch: np.ndarray) -> np.ndarray:
    """Counter index of element (source, kv head, position, channel)."""
    base = (np.uint64(src) * np.uint64(KVH_SLOTS) + np.uint64(kvh)) << np.uint64(POS_BITS)
    p = np.asarray(pos, dtype=np.uint64)
    c = np.asarray(ch, dtype=np.uint64)
    return ((base + p) << np.uint64(7)) + c


def kv_tokens_f32(seed: int, which: str, src: int, kvh: int, pos0: int, n: int,
                  scale: np.ndarray) -> np.ndarray:
    """Raw float32 K or V tokens [n][128] of one (source, kv head) at
    positions pos0 .. pos0+n-1, outlier multipliers applied (exact in fp32)."""
    stream = STREAM_K_CACHE if which == "k" else STREAM_V_CACHE
    key = stream_key(seed, stream)
    pos = np.arange(pos0, pos0 + n, dtype=np.uint64)[:, None]
    ch = np.arange(128, dtype=np.uint64)[None, :]
    x = normal_f32(key, cache_index(src, kvh, pos, ch))
    return (x * np.asarray(scale, dtype=np.float32)[None, :]).astype(np.float32)


def kv_tokens_bf16(seed: int, which: str, src: int, kvh: int, pos0: int, n: int,
                   scale: np.ndarray) -> np.ndarray:
    """As :func:`kv_tokens_f32`, rounded to bfloat16 bit patterns (uint16)."""
    return bf16_bits(kv_tokens_f32(seed, which, src, kvh, pos0, n, scale))


def queries_bf16(seed: int, step: int, batch: int, num_q_heads: int,
                 sigma: np.ndarray) -> np.ndarray:
    """Decode queries for one step, bf16 bits [B][Hq][128]:
    q = sigma * N(0, 1), computed in float64 and rounded via float32."""
    key = stream_key(seed, STREAM_QUERY)
    n = batch * num_q_heads * 128
    base = np.uint64(step) * np.uint64(1 << 24)
    z = normal_f32(key, base + np.arange(n, dtype=np.uint64)).astype(np.float64)
    q = z.reshape(batch, num_q_heads, 128) * sigma[None, :, :]
    return bf16_bits(q.astype(np.float32))


def calibration_tokens(seed: int, n_tokens: int, num_q_heads: int, num_kv_heads: int,
                       sigma: np.ndarray, k_scale: np.ndarray, v_scale: np.ndarray):
    """Calibration sequence of ``n_tokens`` positions, float32:
    q [N][Hq][128] (sigma * N(0,1)), k and v [N][Hkv][128] (N(0,1) times the
    outlier multipliers).  Drawn from streams separate from the cache."""
    kq = stream_key(seed, STREAM_CAL_Q)
    kk = stream_key(seed, STREAM_CAL_K)
    kv = stream_key(seed, STREAM_CAL_V)
    nq = n_tokens * num_q_heads * 128
    nk = n_tokens * num_kv_heads * 128
    q = normal_f32(kq, np.arange(nq, dtype=np.uint64)).reshape(n_tokens, num_q_heads, 128)
    q = (q.astype(np.float64) * sigma[None]).astype(np.float32)
    k = normal_f32(kk, np.arange(nk, dtype=np.uint64)).reshape(n_tokens, num_kv_heads, 128)
    v = normal_f32(kv, np.arange(nk, dtype=np.uint64)).reshape(n_tokens, num_kv_heads, 128)
    k = (k * k_scale[None]).astype(np.float32)
    v = (v * v_scale[None]).astype(np.float32)
    return q, k, v


# ---------------------------------------------------------------------------
# Paging and lengths
# ---------------------------------------------------------------------------

def permutation(seed: int, n: int, stream: int = STREAM_PAGES) -> np.ndarray:
    """Seeded Fisher-Yates permutation of 0..n-1 (int32)."""
    key = stream_key(seed, stream)
    draws = rand64(key, np.arange(n, dtype=np.uint64))
    perm = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = int(draws[i] % np.uint64(i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm.astype(np.int32)


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths drawn uniformly from lo..hi (inclusive), int32 [B]."""
    key = stream_key(seed, STREAM_LENS)
    draws = rand64(key, np.arange(batch, dtype=np.uint64))
    return (lo + (draws % np.uint64(hi - lo + 1)).astype(np.int64)).astype(np.int32)
