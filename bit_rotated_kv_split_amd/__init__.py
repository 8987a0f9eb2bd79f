"""OSCAR INT2 KV-cache decode path for MI355X (gfx950).

The compute lives in ``liboscar.so`` (HIP kernels behind the C ABI of
``include/oscar.h``); this package only marshals arguments to it.  Importing
the package does not load the library; the first call does, and raises if
the library has not been built (there is no fallback path).
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    HEAD_DIM,
    OSCAR_EHIP,
    OSCAR_EINVAL,
    OSCAR_EUNSUPPORTED,
    OSCAR_OK,
    PAGE,
    RECENT,
    SINK,
    OscarCache,
    OscarDims,
    OscarError,
    OscarRotation,
    lib,
    make_cache,
    make_dims,
    make_rotation,
    oscar_block_bytes,
    oscar_calibrate,
    oscar_calibrate_max_tokens,
    oscar_calibrate_workspace_bytes,
    oscar_decode,
    oscar_decode_attn,
    oscar_decode_step,
    oscar_decode_workspace_bytes,
    oscar_history_kernel_for,
    oscar_history_splits,
    oscar_kv_demote,
    oscar_kv_fill_history,
    oscar_last_error,
    oscar_merge_lse,
    oscar_read_history_schedule,
    oscar_set_history_events,
    oscar_set_history_kernel,
    oscar_set_history_target,
)
