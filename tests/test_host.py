"""Host-side checks that need no GPU: the library loads, exports every
function include/oscar.h declares, and rejects bad arguments before it
enqueues anything."""
import ctypes
import os
import re

import pytest

import bit_rotated_kv_split_amd as ok
from bit_rotated_kv_split_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    """Functions declared by every header under include/."""
    names = set()
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_loads_and_exports_every_declared_symbol():
    lib = ok.lib()
    decl = declared_functions()
    assert len(decl) >= 10
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(_lib.EXPORTED) == decl


def test_block_bytes():
    assert ok.oscar_block_bytes(128) == 4608
    assert ok.oscar_block_bytes(64) == 5120
    assert ok.oscar_block_bytes(32) == 6144
    assert ok.oscar_block_bytes(16) == 0


def test_workspace_and_splits():
    d = ok.make_dims(32, 8, 128)
    tgt = lambda n: ok.make_options(history_target=n)   # noqa: E731
    # target 2048 -> 2048 / 8 splits per KV head, plus the batch
    s = ok.oscar_history_splits(d, 32, 100_000, tgt(2048))
    assert s == 256 + 32
    assert ok.oscar_history_splits(d, 32, 1000, tgt(2048)) == s        # lengths decide on the device
    # partials for 8192 / 8 + B history splits and five bf16 chunks per head
    assert ok.oscar_decode_workspace_bytes(d, 32, 100_000) >= (1056 * 32 + 32 * 32 * 5) * 129 * 4
    assert ok.oscar_history_splits(d, 32, 100_000, tgt(64)) == 8 + 32
    assert ok.oscar_history_splits(d, 2, 100_000, tgt(1)) == 1 + 2
    assert ok.oscar_history_splits(ok.make_dims(64, 8, 128), 4, 1000, tgt(1536)) == 192 + 4
    # the layout does not follow the target
    assert ok.oscar_decode_workspace_bytes(d, 32, 100_000) == ok.oscar_decode_workspace_bytes(d, 32, 10)
    for bad_target in (-1, 8193):
        assert ok.oscar_history_splits(d, 2, 1000, tgt(bad_target)) == -1
        assert "history_target" in ok.oscar_last_error()
    bad = ok.make_dims(32, 8, 128, head_dim=64)
    assert ok.oscar_decode_workspace_bytes(bad, 1, 1000) == 0
    assert ok.oscar_history_splits(bad, 1, 1000, tgt(2048)) == -1


def test_default_target_needs_a_device_here():
    """The default target is read from the current device's compute units;
    with no HIP device (this CPU-only host) the sizing call says so instead
    of assuming a chip."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a HIP device is present (covered by the GPU tests)")
    assert ok.oscar_history_splits(ok.make_dims(32, 8, 128), 32, 100_000) == -1
    assert "device" in ok.oscar_last_error()


def test_invalid_options_are_rejected_before_anything_runs():
    d = ok.make_dims(4, 2, 64)
    for o in (ok.make_options(history_kernel=7), ok.make_options(history_kernel=-1),
              ok.make_options(history_target=-5), ok.make_options(history_target=9000)):
        with pytest.raises(ok.OscarError) as e:
            ok.oscar_decode_attn(d, _rot(), _cache(batch=0), None, 100, None, 0, 0, options=o)
        assert e.value.code == ok.OSCAR_EINVAL
        with pytest.raises(ok.OscarError):
            ok.oscar_decode_step(d, _rot(), _cache(batch=0), None, None, None, 100, None, 0, None, None, 0,
                                 options=o)
        assert ok.oscar_history_kernel_for(d, o) == -1
    # the bf16 baseline has a single history kernel
    with pytest.raises(ok.OscarError):
        ok.oscar_bf16_decode(d, ok.make_bf16_cache(0, 0, 0, 0, 0, 0), None, 100, None, 0, None, None, 0,
                             options=ok.make_options(history_kernel=1))
    # valid options on an empty batch: nothing to do, no device needed
    ok.oscar_decode(d, _rot(), _cache(batch=0), None, 100, None, 0, None, None, 0,
                    options=ok.make_options(history_kernel=1, history_target=64))


def _cache(batch=1):
    fake = 0x1000
    return ok.make_cache(fake, 4, fake, fake, fake, fake, fake, 4, fake, batch)


def _rot():
    fake = 0x1000
    return ok.make_rotation(fake, fake, fake, fake)


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, ok.OSCAR_EUNSUPPORTED),
    ("group_size", 16, ok.OSCAR_EUNSUPPORTED),
    ("page_size", 32, ok.OSCAR_EUNSUPPORTED),
    ("sink_len", 32, ok.OSCAR_EUNSUPPORTED),
    ("recent_len", 128, ok.OSCAR_EUNSUPPORTED),
    ("num_kv_heads", 0, ok.OSCAR_EINVAL),
    ("num_q_heads", 12, ok.OSCAR_EINVAL),     # not a multiple of 8
    ("codebook", 2, ok.OSCAR_EUNSUPPORTED),
    ("codebook", -1, ok.OSCAR_EUNSUPPORTED),
])
def test_invalid_dims_rejected(field, value, code):
    d = ok.make_dims(32, 8, 128)
    setattr(d, field, value)
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_kv_demote(d, _rot(), _cache(), None, None, 0)
    assert e.value.code == code
    assert ok.oscar_last_error() != ""


def test_too_many_query_heads_per_kv_head():
    d = ok.make_dims(72, 8, 128)
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_decode_attn(d, _rot(), _cache(), 0x1000, 1000, 0x1000, 1 << 30, 0)
    assert e.value.code == ok.OSCAR_EUNSUPPORTED


def test_null_and_inconsistent_arguments():
    d = ok.make_dims(4, 2, 64)
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_kv_demote(d, _rot(), _cache(), 0x1000, None, 0)
    assert e.value.code == ok.OSCAR_EINVAL
    with pytest.raises(ok.OscarError):
        ok.oscar_decode_attn(d, ok.make_rotation(0, 0x1000, 0x1000, 0x1000), _cache(), 0x1000, 100,
                             0x1000, 1 << 30, 0)
    # workspace too small
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_decode_attn(d, _rot(), _cache(), 0x1000, 100, 0x1000, 16, 0)
    assert e.value.code == ok.OSCAR_EINVAL and "workspace" in ok.oscar_last_error()
    # misaligned workspace
    with pytest.raises(ok.OscarError):
        ok.oscar_decode_attn(d, _rot(), _cache(), 0x1000, 100, 0x1008, 1 << 30, 0)
    # history longer than the page table allows (4 pages = 256 history tokens)
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_decode_attn(d, _rot(), _cache(), 0x1000, 320 + 257, 0x1000, 1 << 30, 0)
    assert "max_pages_per_req" in ok.oscar_last_error()
    # fill outside the batch or beyond the page table
    with pytest.raises(ok.OscarError):
        ok.oscar_kv_fill_history(d, _rot(), _cache(), 1, 0, 10, 0x1000, 0x1000, 0)
    with pytest.raises(ok.OscarError):
        ok.oscar_kv_fill_history(d, _rot(), _cache(), 0, 250, 10, 0x1000, 0x1000, 0)
    # read-back outside the batch, beyond the page table, or with no outputs
    with pytest.raises(ok.OscarError):
        ok.oscar_kv_read_history(d, _cache(), 1, 0, 10, 0x1000, 0x1000, 0)
    with pytest.raises(ok.OscarError):
        ok.oscar_kv_read_history(d, _cache(), 0, 250, 10, 0x1000, 0x1000, 0)
    with pytest.raises(ok.OscarError):
        ok.oscar_kv_read_history(d, _cache(), 0, 0, 10, None, 0x1000, 0)
    with pytest.raises(ok.OscarError):
        ok.oscar_merge_lse(d, _rot(), 1, 100, None, 1 << 30, 0x1000, None, 0)
    # fused decode needs an output
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_decode(d, _rot(), _cache(), 0x1000, 100, 0x1000, 1 << 30, None, None, 0)
    assert e.value.code == ok.OSCAR_EINVAL and "out" in ok.oscar_last_error()
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_decode_step(d, _rot(), _cache(), 0x1000, None, 0x1000, 100, 0x1000, 1 << 30, 0x1000, None, 0)
    assert e.value.code == ok.OSCAR_EINVAL and "k_new" in ok.oscar_last_error()


def test_empty_batch_and_zero_tokens_are_no_ops():
    d = ok.make_dims(4, 2, 64)
    ok.oscar_kv_demote(d, _rot(), _cache(batch=0), None, None, 0)
    ok.oscar_decode_attn(d, _rot(), _cache(batch=0), None, 100, None, 0, 0)
    ok.oscar_merge_lse(d, _rot(), 0, 100, None, 0, None, None, 0)
    ok.oscar_decode(d, _rot(), _cache(batch=0), None, 100, None, 0, None, None, 0)
    ok.oscar_decode_step(d, _rot(), _cache(batch=0), None, None, None, 100, None, 0, None, None, 0)
    ok.oscar_kv_fill_history(d, _rot(), _cache(), 0, 0, 0, None, None, 0)


def test_noalloc_step_rejects_a_batch_beyond_its_scratch():
    """The no-allocation step refuses, on the host, a batch whose workspace
    would not fit the library's 64 MiB scratch (64 q heads over 8 KV
    heads: more than 111 requests), and an empty batch is a no-op."""
    d = ok.make_dims(64, 8, 128)
    assert ok.oscar_decode_workspace_bytes(d, 111, 131_072) <= ok.NOALLOC_SCRATCH_BYTES
    assert ok.oscar_decode_workspace_bytes(d, 112, 131_072) > ok.NOALLOC_SCRATCH_BYTES
    fake = 0x1000
    big = ok.make_cache(fake, 4, fake, fake, fake, fake, fake, 4, fake, 112)
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_decode_step_noalloc(d, _rot(), big, fake, fake, fake, 100, fake, None, 0)
    assert e.value.code == ok.OSCAR_EINVAL and "scratch" in ok.oscar_last_error()
    ok.oscar_decode_step_noalloc(d, _rot(), _cache(batch=0), None, None, None, 100, None, None, 0)


def test_probe_rejects_misaligned_buffers():
    for buf, n in ((0x1001, 4096), (0x1000, 4095), (0, 4096)):
        with pytest.raises(ok.OscarError) as e:
            ok.oscar_probe_read(buf, n, True, 0x1000, 0)
        assert e.value.code == ok.OSCAR_EINVAL
    ok.oscar_probe_read(0x1000, 0, False, 0x1000, 0)    # nothing to read
    for buf, n, waves in ((0x1001, 8192, 2), (0x1000, 8192 + 16, 2), (0x1000, 4096, 2), (0x1000, 8192, 0),
                          (0, 8192, 2)):
        with pytest.raises(ok.OscarError) as e:
            ok.oscar_probe_read_blocks(buf, n, True, waves, 0x1000, 0)
        assert e.value.code == ok.OSCAR_EINVAL
    ok.oscar_probe_read_blocks(0x1000, 0, True, 4, 0x1000, 0)   # nothing to read


def test_history_kernel_selector():
    d = ok.make_dims(32, 8, 128)
    assert ok.oscar_history_kernel_for(d) == 2
    assert ok.oscar_history_kernel_for(d, ok.make_options(history_kernel=1)) == 1
    assert ok.oscar_history_kernel_for(d, ok.make_options(history_kernel=2)) == 2
    assert ok.oscar_history_kernel_for(d, ok.make_options(history_kernel=7)) == -1


def test_codebook_constants_equal_the_oracle():
    """The library's Lloyd-Max codebook (bisection on the threshold) and the
    oracle's (Lloyd's alternation) agree to the last float32 bit."""
    import numpy as np
    from oracle import oscar as O
    lev, thr = ok.oscar_codebook(ok.CODEBOOK_LLOYD_MAX)
    olev, othr = O.lloyd_max_codebook()
    assert lev.view(np.uint32).tolist() == olev.view(np.uint32).tolist()
    assert thr.view(np.uint32).tolist() == othr.view(np.uint32).tolist()
    lev, thr = ok.oscar_codebook(ok.CODEBOOK_UNIFORM)
    assert lev.tolist() == [0, 1, 2, 3] and thr.tolist() == [0.5, 1.5, 2.5]
    with pytest.raises(ok.OscarError):
        ok.oscar_codebook(5)


def test_history_kernel_choice_by_codebook_and_group():
    """The matrix-core kernel covers every supported group size and both
    codebooks; the selector still forces the vector-ALU one."""
    for g in (32, 64, 128):
        for cb in (ok.CODEBOOK_UNIFORM, ok.CODEBOOK_LLOYD_MAX):
            for hq in (8, 32, 64):
                assert ok.oscar_history_kernel_for(ok.make_dims(hq, 8, g, codebook=cb)) == 2
    assert ok.oscar_history_kernel_for(ok.make_dims(32, 8, 32, codebook=ok.CODEBOOK_LLOYD_MAX),
                                       ok.make_options(history_kernel=1)) == 1


def test_last_error_is_thread_local():
    import threading
    d = ok.make_dims(32, 8, 128, head_dim=64)
    with pytest.raises(ok.OscarError):
        ok.oscar_kv_demote(d, _rot(), _cache(), None, None, 0)
    seen = []
    t = threading.Thread(target=lambda: seen.append(ok.oscar_last_error()))
    t.start()
    t.join()
    assert seen == [""] and "head_dim" in ok.oscar_last_error()


def test_bf16_baseline_host_checks():
    d = ok.make_dims(32, 8, 128)
    assert ok.oscar_bf16_block_bytes() == 2 * 64 * 128 * 2
    assert ok.oscar_bf16_decode_workspace_bytes(d, 32) >= (1024 + 32) * 32 * 129 * 4
    fake = 0x1000
    c = ok.make_bf16_cache(fake, 10, fake, 4, fake, 2)
    with pytest.raises(ok.OscarError) as e:   # 300 positions need 5 pages > 4
        ok.oscar_bf16_decode(d, c, fake, 300, fake, 1 << 30, fake, None, 0)
    assert e.value.code == ok.OSCAR_EINVAL and "max_pages_per_req" in ok.oscar_last_error()
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_bf16_decode(d, c, fake, 100, fake, 16, fake, None, 0)
    assert e.value.code == ok.OSCAR_EINVAL and "workspace" in ok.oscar_last_error()
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_bf16_fill(d, c, 2, 0, 10, fake, fake, 0)
    assert e.value.code == ok.OSCAR_EINVAL and "request" in ok.oscar_last_error()
    with pytest.raises(ok.OscarError) as e:
        ok.oscar_bf16_fill(d, c, 0, 250, 10, fake, fake, 0)
    assert e.value.code == ok.OSCAR_EINVAL
    with pytest.raises(ok.OscarError):
        ok.oscar_bf16_append(d, c, None, fake, 0)
    empty = ok.make_bf16_cache(fake, 10, fake, 4, fake, 0)
    ok.oscar_bf16_decode(d, empty, None, 100, None, 0, None, None, 0)
