"""ctypes binding of the plain C++ oracle (``oracle/oscar_ref.cpp``).

TEST INFRASTRUCTURE ONLY, like the numpy oracle: only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use
it.  The library is built with the host compiler (g++ -O3 -fopenmp, no
machine-specific flags) into ``oracle/liboscar_oracle.so``; it shares no
source with the HIP library.  The arrays passed in are numpy arrays on the
host; this module only marshals them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oscar_ref.cpp")
LIB = os.path.join(HERE, "liboscar_oracle.so")
CODEBOOKS = {"uniform": 0, "lloyd-max": 1}

_lib = None


def build() -> str:
    """Compile the oracle library (always; a few seconds)."""
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O3", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra", SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


class Pair(ctypes.Structure):
    """One (request, KV head) pair; mirrors OscarOraclePair."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("len", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("r_k", ctypes.c_void_p), ("r_v", ctypes.c_void_p),
                ("clip_k", ctypes.c_void_p), ("clip_v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


def lib():
    """The loaded library, built first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.oscar_oracle_lloyd_max.argtypes = [vp, vp]
        L.oscar_oracle_demote.argtypes = [vp, i64, vp, vp, i32, i32, vp, vp, vp]
        L.oscar_oracle_attend_pairs.argtypes = [vp, i32, i32, i32, i32, i32]
        for f in (L.oscar_oracle_lloyd_max, L.oscar_oracle_demote, L.oscar_oracle_attend_pairs):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"{what}: error {rc}")


def lloyd_max():
    """Float64 levels [4] and thresholds [3] of the N(0, 1) Lloyd-Max quantizer."""
    lev = np.zeros(4)
    thr = np.zeros(3)
    _check(lib().oscar_oracle_lloyd_max(_ptr(lev), _ptr(thr)), "lloyd_max")
    return lev, thr


def demote(x_bits, r32, clip32, group: int, codebook: str = "uniform"):
    """Codes uint8 [n][128], scale and zero float32 [n][128/group] of n bf16
    tokens of one KV head (same contract as the numpy oracle's demote)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16).reshape(-1, 128)
    r = np.ascontiguousarray(r32, dtype=np.float32)
    c = np.ascontiguousarray(clip32, dtype=np.float32)
    if r.shape != (128, 128) or c.shape != (128,):
        raise ValueError("rotation must be [128][128] and clip [128]")
    n = x.shape[0]
    codes = np.zeros((n, 128), np.uint8)
    s = np.zeros((n, 128 // group), np.float32)
    z = np.zeros((n, 128 // group), np.float32)
    _check(lib().oscar_oracle_demote(_ptr(x), n, _ptr(r), _ptr(c), group, CODEBOOKS[codebook],
                                     _ptr(codes), _ptr(s), _ptr(z)), "demote")
    return codes, s, z


def attend_pairs(pairs, g: int, group: int, codebook: str = "uniform", threads: int = 1):
    """Run prepared (request, KV head) pairs on `threads` OpenMP threads.

    Each pair is a dict: q [g][128] bf16 bits; k and v, matching C-contiguous
    uint16 arrays [L][stride] whose rows hold the head's token at element
    offset ``off`` (default 0); r_k, r_v [128][128] and clip_k, clip_v [128]
    float32.  Returns [(out [g][128], lse [g])] in the pairs' order."""
    arr = (Pair * max(1, len(pairs)))()
    keep, results = [], []
    for i, p in enumerate(pairs):
        q = np.ascontiguousarray(p["q"], dtype=np.uint16).reshape(g, 128)
        k, v, off = p["k"], p["v"], int(p.get("off", 0))
        if k.dtype != np.uint16 or v.dtype != np.uint16 or k.shape != v.shape or k.ndim != 2:
            raise ValueError("k and v must be matching [L][stride] uint16 arrays")
        if not (k.flags.c_contiguous and v.flags.c_contiguous) or off < 0 or off + 128 > k.shape[1]:
            raise ValueError("k and v rows must be contiguous and hold the head at [off, off + 128)")
        mats = [np.ascontiguousarray(p[n], dtype=np.float32) for n in ("r_k", "r_v", "clip_k", "clip_v")]
        if mats[0].shape != (128, 128) or mats[1].shape != (128, 128) or mats[2].shape != (128,) \
                or mats[3].shape != (128,):
            raise ValueError("rotations must be [128][128] and clips [128]")
        out = np.zeros((g, 128))
        lse = np.zeros(g)
        arr[i] = Pair(_ptr(q), _ptr(k) + 2 * off, _ptr(v) + 2 * off, k.shape[0], k.shape[1],
                      _ptr(mats[0]), _ptr(mats[1]), _ptr(mats[2]), _ptr(mats[3]), _ptr(out), _ptr(lse))
        keep.append((q, k, v, mats))
        results.append((out, lse))
    _check(lib().oscar_oracle_attend_pairs(ctypes.addressof(arr), len(pairs), g, group,
                                           CODEBOOKS[codebook], threads), "attend_pairs")
    return results


def request_attention(q_bits, k_tokens, v_tokens, r_k32, r_v32, clip_k, clip_v, group: int,
                      codebook: str = "uniform", threads: int = 1):
    """Same contract as the numpy oracle's request_attention: q_bits
    [Hq][128], k_tokens/v_tokens [L][Hkv][128] bf16 bits, rotations
    [Hkv][128][128], clips [Hkv][128].  Returns out [Hq][128], lse [Hq]."""
    k_tokens = np.ascontiguousarray(k_tokens, dtype=np.uint16)
    v_tokens = np.ascontiguousarray(v_tokens, dtype=np.uint16)
    L, hkv = k_tokens.shape[0], k_tokens.shape[1]
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    g = q_bits.shape[0] // hkv
    k = k_tokens.reshape(L, hkv * 128)
    v = v_tokens.reshape(L, hkv * 128)
    pairs = [{"q": q_bits[j * g:(j + 1) * g], "k": k, "v": v, "off": j * 128, "r_k": r_k32[j],
              "r_v": r_v32[j], "clip_k": clip_k[j], "clip_v": clip_v[j]} for j in range(hkv)]
    res = attend_pairs(pairs, g, group, codebook, threads)
    out = np.concatenate([o for o, _ in res], axis=0)
    lse = np.concatenate([s for _, s in res], axis=0)
    return out, lse
