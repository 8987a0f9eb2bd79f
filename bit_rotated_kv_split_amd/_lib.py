"""ctypes binding of liboscar.so (the C ABI declared in include/oscar.h).

Argument marshalling only: every computation runs in the HIP library.  The
functions carry the C names and raise :class:`OscarError` on a non-zero
return code.  Tensors are torch tensors on the GPU (or raw device addresses
as ints); the library neither keeps nor frees them.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liboscar.so")

OSCAR_OK = 0
OSCAR_EINVAL = 1
OSCAR_EUNSUPPORTED = 2
OSCAR_EHIP = 3

CODEBOOK_UNIFORM = 0
CODEBOOK_LLOYD_MAX = 1

HEAD_DIM = 128
PAGE = 64
SINK = 64
RECENT = 256


class OscarError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"oscar error {code}: {msg}")
        self.code = code


class OscarDims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("sink_len", ctypes.c_int32),
                ("recent_len", ctypes.c_int32), ("codebook", ctypes.c_int32)]


class OscarRotation(ctypes.Structure):
    _fields_ = [("r_k", ctypes.c_void_p), ("r_v", ctypes.c_void_p),
                ("clip_k", ctypes.c_void_p), ("clip_v", ctypes.c_void_p)]


class OscarCache(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("n_pages", ctypes.c_int64),
                ("sink_k", ctypes.c_void_p), ("sink_v", ctypes.c_void_p),
                ("recent_k", ctypes.c_void_p), ("recent_v", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("max_pages_per_req", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("batch", ctypes.c_int32)]


class OscarBf16Cache(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("n_pages", ctypes.c_int64),
                ("page_table", ctypes.c_void_p), ("max_pages_per_req", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("batch", ctypes.c_int32)]


class OscarDecodeOptions(ctypes.Structure):
    _fields_ = [("history_kernel", ctypes.c_int32), ("history_target", ctypes.c_int32),
                ("history_start_event", ctypes.c_void_p), ("history_stop_event", ctypes.c_void_p),
                ("history_clock_trace", ctypes.c_void_p)]


# (name, restype, argtypes) of every exported function
_P = ctypes.POINTER
_SIGS = [
    ("oscar_block_bytes", ctypes.c_size_t, [ctypes.c_int32]),
    ("oscar_codebook", ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    ("oscar_kv_demote", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), _P(OscarCache),
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("oscar_kv_fill_history", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), _P(OscarCache),
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("oscar_kv_read_history", ctypes.c_int, [_P(OscarDims), _P(OscarCache), ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("oscar_history_splits", ctypes.c_int32, [_P(OscarDims), ctypes.c_int32, ctypes.c_int32]),
    ("oscar_history_splits_ex", ctypes.c_int32, [_P(OscarDims), ctypes.c_int32, ctypes.c_int32,
                                                 _P(OscarDecodeOptions)]),
    ("oscar_decode_workspace_bytes", ctypes.c_size_t, [_P(OscarDims), ctypes.c_int32, ctypes.c_int32]),
    ("oscar_decode_attn", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), _P(OscarCache),
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    ("oscar_decode_attn_ex", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), _P(OscarCache),
                                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_size_t, _P(OscarDecodeOptions), ctypes.c_void_p]),
    ("oscar_decode", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), _P(OscarCache),
                                    ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("oscar_decode_ex", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), _P(OscarCache),
                                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p, ctypes.c_void_p, _P(OscarDecodeOptions),
                                       ctypes.c_void_p]),
    ("oscar_decode_step", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), _P(OscarCache),
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]),
    ("oscar_decode_step_ex", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), _P(OscarCache),
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                            _P(OscarDecodeOptions), ctypes.c_void_p]),
    ("oscar_decode_step_noalloc", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), _P(OscarCache),
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p]),
    ("oscar_merge_lse", ctypes.c_int, [_P(OscarDims), _P(OscarRotation), ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("oscar_calibrate_max_tokens", ctypes.c_int32, []),
    ("oscar_calibrate_workspace_bytes", ctypes.c_size_t, [_P(OscarDims), ctypes.c_int32]),
    ("oscar_calibrate", ctypes.c_int, [_P(OscarDims), ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("oscar_read_history_schedule", ctypes.c_int, [_P(OscarDims), ctypes.c_int32, ctypes.c_void_p,
                                                   ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_int32, ctypes.c_void_p]),
    ("oscar_bf16_block_bytes", ctypes.c_size_t, []),
    ("oscar_bf16_fill", ctypes.c_int, [_P(OscarDims), _P(OscarBf16Cache), ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    ("oscar_bf16_append", ctypes.c_int, [_P(OscarDims), _P(OscarBf16Cache), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]),
    ("oscar_bf16_decode_workspace_bytes", ctypes.c_size_t, [_P(OscarDims), ctypes.c_int32]),
    ("oscar_bf16_decode", ctypes.c_int, [_P(OscarDims), _P(OscarBf16Cache), ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]),
    ("oscar_bf16_decode_ex", ctypes.c_int, [_P(OscarDims), _P(OscarBf16Cache), ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                            _P(OscarDecodeOptions), ctypes.c_void_p]),
    ("oscar_history_kernel_for", ctypes.c_int, [_P(OscarDims), _P(OscarDecodeOptions)]),
    ("oscar_last_error", ctypes.c_char_p, []),
    ("oscar_probe_read", ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    ("oscar_probe_read_blocks", ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_void_p, ctypes.c_void_p]),
]
EXPORTED = [s[0] for s in _SIGS]

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise OscarError(OSCAR_EHIP, f"{LIB_PATH} is missing; run "
                                 "`python -m bit_rotated_kv_split_amd.build` first")
            handle = ctypes.CDLL(LIB_PATH)
            for name, res, args in _SIGS:
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
        return _lib


def _ptr(x) -> int | None:
    """Device address of a tensor (or an int address, or None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != OSCAR_OK:
        raise OscarError(rc, lib().oscar_last_error().decode())


# ------------------------------------------------------------------ structs

def make_dims(num_q_heads: int, num_kv_heads: int, group_size: int, head_dim: int = HEAD_DIM,
              page_size: int = PAGE, sink_len: int = SINK, recent_len: int = RECENT,
              codebook: int = CODEBOOK_UNIFORM) -> OscarDims:
    return OscarDims(num_q_heads, num_kv_heads, head_dim, group_size, page_size, sink_len, recent_len,
                     codebook)


def oscar_codebook(codebook: int):
    """(levels float32 [4], thresholds float32 [3]) of a codebook, from the library."""
    import numpy as np
    lev = np.zeros(4, dtype=np.float32)
    thr = np.zeros(3, dtype=np.float32)
    rc = lib().oscar_codebook(codebook, lev.ctypes.data, thr.ctypes.data)
    if rc != OSCAR_OK:
        raise OscarError(rc, f"codebook {codebook}")
    return lev, thr


def _event_handle(ev):
    """hipEvent_t of a HipEvent-like object (``.ptr``), a torch event
    (``.cuda_event``) or an int; None stays None."""
    if ev is None:
        return None
    if hasattr(ev, "ptr"):
        return ev.ptr
    if hasattr(ev, "cuda_event"):
        return ev.cuda_event
    return ev


def make_options(history_kernel: int = 0, history_target: int = 0, start_event=None,
                 stop_event=None, clock_trace=None) -> OscarDecodeOptions:
    """Per-call options of the decode entry points (oscar_decode_options);
    clock_trace: a device uint64 [4] tensor or address, or None."""
    o = OscarDecodeOptions(history_kernel, history_target, _event_handle(start_event), _event_handle(stop_event),
                           _ptr(clock_trace))
    o._keep = (start_event, stop_event, clock_trace)
    return o


def wall_clock_khz(device: int = 0) -> int:
    """The device's constant-rate counter frequency in kHz
    (hipDeviceAttributeWallClockRate, value 10017 of hipDeviceAttribute_t
    in hip_runtime_api.h), for history_clock_trace readings."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    hip.hipDeviceGetAttribute.restype = ctypes.c_int
    v = ctypes.c_int()
    rc = hip.hipDeviceGetAttribute(ctypes.byref(v), 10017, device)
    if rc != 0:
        raise OscarError(OSCAR_EHIP, f"hipDeviceGetAttribute(wall clock rate) failed ({rc})")
    return v.value


def _opt(options):
    return None if options is None else ctypes.byref(options)


def make_rotation(r_k, r_v, clip_k, clip_v) -> OscarRotation:
    rot = OscarRotation(_ptr(r_k), _ptr(r_v), _ptr(clip_k), _ptr(clip_v))
    rot._keep = (r_k, r_v, clip_k, clip_v)
    return rot


def make_cache(pages, n_pages: int, sink_k, sink_v, recent_k, recent_v, page_table,
               max_pages_per_req: int, seq_lens, batch: int) -> OscarCache:
    c = OscarCache(_ptr(pages), n_pages, _ptr(sink_k), _ptr(sink_v), _ptr(recent_k),
                   _ptr(recent_v), _ptr(page_table), max_pages_per_req, _ptr(seq_lens), batch)
    c._keep = (pages, sink_k, sink_v, recent_k, recent_v, page_table, seq_lens)
    return c


def make_bf16_cache(pages, n_pages: int, page_table, max_pages_per_req: int, seq_lens,
                    batch: int) -> OscarBf16Cache:
    c = OscarBf16Cache(_ptr(pages), n_pages, _ptr(page_table), max_pages_per_req, _ptr(seq_lens), batch)
    c._keep = (pages, page_table, seq_lens)
    return c


# ------------------------------------------------------------- entry points

def oscar_block_bytes(group_size: int) -> int:
    return lib().oscar_block_bytes(group_size)


def oscar_kv_demote(dims, rot, cache, k_new, v_new, stream=None) -> None:
    _check(lib().oscar_kv_demote(ctypes.byref(dims), ctypes.byref(rot), ctypes.byref(cache),
                                 _ptr(k_new), _ptr(v_new), _stream(stream)))


def oscar_kv_fill_history(dims, rot, cache, request: int, hist_begin: int, n_tokens: int,
                          k_tokens, v_tokens, stream=None) -> None:
    _check(lib().oscar_kv_fill_history(ctypes.byref(dims), ctypes.byref(rot), ctypes.byref(cache),
                                       request, hist_begin, n_tokens, _ptr(k_tokens),
                                       _ptr(v_tokens), _stream(stream)))


def oscar_kv_read_history(dims, cache, request: int, hist_begin: int, n_tokens: int, k_out, v_out,
                          stream=None) -> None:
    _check(lib().oscar_kv_read_history(ctypes.byref(dims), ctypes.byref(cache), request, hist_begin, n_tokens,
                                       _ptr(k_out), _ptr(v_out), _stream(stream)))


def oscar_history_splits(dims, batch: int, max_seq_len: int, options=None) -> int:
    if options is None:
        return lib().oscar_history_splits(ctypes.byref(dims), batch, max_seq_len)
    return lib().oscar_history_splits_ex(ctypes.byref(dims), batch, max_seq_len, _opt(options))


def oscar_decode_workspace_bytes(dims, batch: int, max_seq_len: int) -> int:
    return lib().oscar_decode_workspace_bytes(ctypes.byref(dims), batch, max_seq_len)


def oscar_decode_attn(dims, rot, cache, q, max_seq_len: int, workspace, workspace_bytes: int,
                      stream=None, options=None) -> None:
    """oscar_decode_attn, or oscar_decode_attn_ex when options are given."""
    args = (ctypes.byref(dims), ctypes.byref(rot), ctypes.byref(cache), _ptr(q), max_seq_len, _ptr(workspace),
            workspace_bytes)
    if options is None:
        _check(lib().oscar_decode_attn(*args, _stream(stream)))
    else:
        _check(lib().oscar_decode_attn_ex(*args, _opt(options), _stream(stream)))


def oscar_decode(dims, rot, cache, q, max_seq_len: int, workspace, workspace_bytes: int, out,
                 lse_out=None, stream=None, options=None) -> None:
    """oscar_decode, or oscar_decode_ex when options are given."""
    args = (ctypes.byref(dims), ctypes.byref(rot), ctypes.byref(cache), _ptr(q), max_seq_len, _ptr(workspace),
            workspace_bytes, _ptr(out), _ptr(lse_out))
    if options is None:
        _check(lib().oscar_decode(*args, _stream(stream)))
    else:
        _check(lib().oscar_decode_ex(*args, _opt(options), _stream(stream)))


def oscar_decode_step(dims, rot, cache, k_new, v_new, q, max_seq_len: int, workspace,
                      workspace_bytes: int, out, lse_out=None, stream=None, options=None) -> None:
    """oscar_decode_step, or oscar_decode_step_ex when options are given."""
    args = (ctypes.byref(dims), ctypes.byref(rot), ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(q),
            max_seq_len, _ptr(workspace), workspace_bytes, _ptr(out), _ptr(lse_out))
    if options is None:
        _check(lib().oscar_decode_step(*args, _stream(stream)))
    else:
        _check(lib().oscar_decode_step_ex(*args, _opt(options), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20


def oscar_decode_step_noalloc(dims, rot, cache, k_new, v_new, q, max_seq_len: int, out, lse_out=None,
                              stream=None) -> None:
    """oscar_decode_step with the library's own per-device scratch as its
    workspace (no allocation anywhere in the call)."""
    _check(lib().oscar_decode_step_noalloc(ctypes.byref(dims), ctypes.byref(rot), ctypes.byref(cache),
                                           _ptr(k_new), _ptr(v_new), _ptr(q), max_seq_len, _ptr(out),
                                           _ptr(lse_out), _stream(stream)))


def oscar_merge_lse(dims, rot, batch: int, max_seq_len: int, workspace, workspace_bytes: int,
                    out, lse_out=None, stream=None) -> None:
    _check(lib().oscar_merge_lse(ctypes.byref(dims), ctypes.byref(rot), batch, max_seq_len,
                                 _ptr(workspace), workspace_bytes, _ptr(out), _ptr(lse_out),
                                 _stream(stream)))


def oscar_calibrate_max_tokens() -> int:
    return lib().oscar_calibrate_max_tokens()


def oscar_calibrate_workspace_bytes(dims, n_tokens: int) -> int:
    return lib().oscar_calibrate_workspace_bytes(ctypes.byref(dims), n_tokens)


def oscar_calibrate(dims, n_tokens: int, q, k, v, clip_percentile: float, r_k, r_v, clip_k, clip_v,
                    r_k_host=None, r_v_host=None, workspace=None, workspace_bytes: int = 0,
                    stream=None) -> None:
    """Device outputs r_k/r_v/clip_k/clip_v; optional host float64 outputs
    given as numpy arrays (written in place)."""
    def host(a):
        if a is None:
            return None
        assert a.dtype.name == "float64" and a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    _check(lib().oscar_calibrate(ctypes.byref(dims), n_tokens, _ptr(q), _ptr(k), _ptr(v),
                                 clip_percentile, _ptr(r_k), _ptr(r_v), _ptr(clip_k), _ptr(clip_v),
                                 host(r_k_host), host(r_v_host), _ptr(workspace), workspace_bytes,
                                 _stream(stream)))


def oscar_read_history_schedule(dims, batch: int, workspace, workspace_bytes: int, stream=None):
    """(splits int32 [n][3] {request, first page, end page}, requests int32
    [batch][2] {first split, count}) of the last decode on this workspace."""
    import numpy as np
    # capacity of the workspace's split table: the largest target's bound
    cap = lib().oscar_history_splits_ex(ctypes.byref(dims), batch, 1,
                                        ctypes.byref(make_options(history_target=8192)))
    splits = np.zeros((max(cap, 1), 3), dtype=np.int32)
    reqs = np.zeros((batch, 2), dtype=np.int32)
    n = lib().oscar_read_history_schedule(ctypes.byref(dims), batch, _ptr(workspace), workspace_bytes,
                                          splits.ctypes.data, reqs.ctypes.data, splits.shape[0],
                                          _stream(stream))
    if n < 0:
        _check(-n)
    return splits[:n].copy(), reqs


def oscar_bf16_block_bytes() -> int:
    return lib().oscar_bf16_block_bytes()


def oscar_bf16_fill(dims, cache, request: int, pos_begin: int, n_tokens: int, k_tokens, v_tokens,
                    stream=None) -> None:
    _check(lib().oscar_bf16_fill(ctypes.byref(dims), ctypes.byref(cache), request, pos_begin, n_tokens,
                                 _ptr(k_tokens), _ptr(v_tokens), _stream(stream)))


def oscar_bf16_append(dims, cache, k_new, v_new, stream=None) -> None:
    _check(lib().oscar_bf16_append(ctypes.byref(dims), ctypes.byref(cache), _ptr(k_new), _ptr(v_new),
                                   _stream(stream)))


def oscar_bf16_decode_workspace_bytes(dims, batch: int) -> int:
    return lib().oscar_bf16_decode_workspace_bytes(ctypes.byref(dims), batch)


def oscar_bf16_decode(dims, cache, q, max_seq_len: int, workspace, workspace_bytes: int, out,
                      lse_out=None, stream=None, options=None) -> None:
    """oscar_bf16_decode, or oscar_bf16_decode_ex when options are given."""
    args = (ctypes.byref(dims), ctypes.byref(cache), _ptr(q), max_seq_len, _ptr(workspace), workspace_bytes,
            _ptr(out), _ptr(lse_out))
    if options is None:
        _check(lib().oscar_bf16_decode(*args, _stream(stream)))
    else:
        _check(lib().oscar_bf16_decode_ex(*args, _opt(options), _stream(stream)))


def oscar_history_kernel_for(dims, options=None) -> int:
    return lib().oscar_history_kernel_for(ctypes.byref(dims), _opt(options))


def oscar_probe_read(buf, nbytes: int, nontemporal: bool, sink, stream=None) -> None:
    """One pass of the HBM read probe over nbytes of buf (include/oscar_probe.h)."""
    _check(lib().oscar_probe_read(_ptr(buf), nbytes, 1 if nontemporal else 0, _ptr(sink), _stream(stream)))


def oscar_probe_read_blocks(buf, nbytes: int, nontemporal: bool, waves: int, sink, stream=None) -> None:
    """One pass of the block-streaming read probe (include/oscar_probe.h)."""
    _check(lib().oscar_probe_read_blocks(_ptr(buf), nbytes, 1 if nontemporal else 0, waves, _ptr(sink),
                                         _stream(stream)))


def oscar_last_error() -> str:
    return lib().oscar_last_error().decode()
