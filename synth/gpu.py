"""ctypes loader of synth/libsynth.so, the GPU twin of the token generator in
synth/gen.py (same draws, bit-identical bf16 output)."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

from . import gen

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libsynth.so")
_lib = None


def build() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_DIR, "fill.hip"), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed building libsynth.so:\n" + res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing; run __graft_entry__.build()")
        h = ctypes.CDLL(LIB_PATH)
        h.synth_fill_kv.restype = ctypes.c_int
        h.synth_fill_kv.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p]
        _lib = h
    return _lib


def fill_kv(dst, n_tok: int, hkv: int, stride_t: int, stride_h: int, seed: int, which: str,
            src: int, pos0: int, scale, stream: int) -> None:
    """Write bf16 tokens of (src, positions pos0..pos0+n_tok-1) for every kv
    head into ``dst`` (a device address or tensor) at
    dst[t*stride_t + h*stride_h + c]; ``scale`` is a device float [Hkv][128]."""
    stream_id = gen.STREAM_K_CACHE if which == "k" else gen.STREAM_V_CACHE
    key = int(gen.stream_key(seed, stream_id))
    d = dst if isinstance(dst, int) else dst.data_ptr()
    s = scale if isinstance(scale, int) else scale.data_ptr()
    rc = lib().synth_fill_kv(d, n_tok, hkv, stride_t, stride_h, key, src, pos0, s, stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_kv failed ({rc})")
