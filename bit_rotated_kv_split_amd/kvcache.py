"""Device buffers of one layer's three-region OSCAR cache, as torch tensors.

torch is used for device memory and streams only; every read or write of
the cache contents happens in the HIP library (``_lib``).
"""
from __future__ import annotations

import torch

from . import _lib


class PagedKVCache:
    """bf16 sink/recent buffers, INT2 history pages, page table and lengths.

    Layouts are those of ``oscar_cache`` in include/oscar.h:
      pages      uint8 [n_pages][Hkv][oscar_block_bytes(G)]
      sink_k/v   bf16  [B][Hkv][64][128]
      recent_k/v bf16  [B][Hkv][256][128] (ring, position p at slot (p-64) % 256)
      page_table int32 [B][max_pages_per_req]
      seq_lens   int32 [B]
    """

    def __init__(self, num_q_heads: int, num_kv_heads: int, group_size: int, batch: int,
                 max_pages_per_req: int, n_pages: int, device: str = "cuda",
                 codebook: int = _lib.CODEBOOK_UNIFORM):
        self.dims = _lib.make_dims(num_q_heads, num_kv_heads, group_size, codebook=codebook)
        self.codebook = codebook
        self.batch = batch
        self.num_q_heads = num_q_heads
        self.num_kv_heads = num_kv_heads
        self.group_size = group_size
        self.max_pages_per_req = max_pages_per_req
        self.n_pages = n_pages
        bb = _lib.oscar_block_bytes(group_size)
        if bb == 0:
            raise _lib.OscarError(_lib.OSCAR_EUNSUPPORTED, f"group size {group_size}")
        self.block_bytes = bb
        self.pages = torch.zeros((max(n_pages, 1), num_kv_heads, bb), dtype=torch.uint8, device=device)
        shape_s = (batch, num_kv_heads, _lib.SINK, _lib.HEAD_DIM)
        shape_r = (batch, num_kv_heads, _lib.RECENT, _lib.HEAD_DIM)
        self.sink_k = torch.zeros(shape_s, dtype=torch.bfloat16, device=device)
        self.sink_v = torch.zeros(shape_s, dtype=torch.bfloat16, device=device)
        self.recent_k = torch.zeros(shape_r, dtype=torch.bfloat16, device=device)
        self.recent_v = torch.zeros(shape_r, dtype=torch.bfloat16, device=device)
        self.page_table = torch.zeros((batch, max(max_pages_per_req, 1)), dtype=torch.int32, device=device)
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, device=device)
        self._struct = None

    def struct(self) -> _lib.OscarCache:
        if self._struct is None:
            self._struct = _lib.make_cache(self.pages, self.n_pages, self.sink_k, self.sink_v,
                                           self.recent_k, self.recent_v, self.page_table,
                                           self.max_pages_per_req, self.seq_lens, self.batch)
        return self._struct


class Bf16PagedCache:
    """The all-bf16 baseline cache (``oscar_bf16_cache`` in include/oscar.h):
      pages      bf16  [n_pages][Hkv][2][64][128]  (keys, then values, of 64 positions)
      page_table int32 [B][max_pages_per_req]      (position p -> page p // 64, row p % 64)
      seq_lens   int32 [B]
    """

    def __init__(self, num_q_heads: int, num_kv_heads: int, batch: int, max_pages_per_req: int,
                 n_pages: int, device: str = "cuda"):
        self.dims = _lib.make_dims(num_q_heads, num_kv_heads, 128)
        self.batch = batch
        self.num_q_heads = num_q_heads
        self.num_kv_heads = num_kv_heads
        self.max_pages_per_req = max_pages_per_req
        self.n_pages = n_pages
        self.pages = torch.zeros((max(n_pages, 1), num_kv_heads, 2, _lib.PAGE, _lib.HEAD_DIM),
                                 dtype=torch.bfloat16, device=device)
        self.page_table = torch.zeros((batch, max(max_pages_per_req, 1)), dtype=torch.int32, device=device)
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, device=device)
        self._struct = None

    def struct(self) -> _lib.OscarBf16Cache:
        if self._struct is None:
            self._struct = _lib.make_bf16_cache(self.pages, self.n_pages, self.page_table,
                                                self.max_pages_per_req, self.seq_lens, self.batch)
        return self._struct


class Rotation:
    """Float32 device copies of R_K, R_V [Hkv][128][128] and clips [Hkv][128]."""

    def __init__(self, r_k, r_v, clip_k, clip_v, device: str = "cuda"):
        def dev(x):
            return torch.as_tensor(x, dtype=torch.float32).contiguous().to(device)
        self.r_k, self.r_v = dev(r_k), dev(r_v)
        self.clip_k, self.clip_v = dev(clip_k), dev(clip_v)
        self.struct = _lib.make_rotation(self.r_k, self.r_v, self.clip_k, self.clip_v)


class DecodeWorkspace:
    """Workspace of one (batch, max_seq_len) decode configuration.  `splits`
    is the split bound of the default schedule on the current device (or of
    the given options')."""

    def __init__(self, dims, batch: int, max_seq_len: int, device: str = "cuda", options=None):
        self.batch = batch
        self.max_seq_len = max_seq_len
        self.nbytes = _lib.oscar_decode_workspace_bytes(dims, batch, max_seq_len)
        if self.nbytes == 0 and batch > 0:
            raise _lib.OscarError(_lib.OSCAR_EINVAL, _lib.oscar_last_error())
        # torch's caching allocator returns 512-byte aligned blocks
        self.buf = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device)
        self.splits = _lib.oscar_history_splits(dims, batch, max_seq_len, options)


def decode_step(cache: PagedKVCache, rot: Rotation, ws: DecodeWorkspace, q, out, lse=None,
                k_new=None, v_new=None, stream=None, options=None) -> None:
    """One decode step on the current stream (oscar_decode_step): demote (and
    append k_new/v_new if given), decode attention, merge.  seq_lens must
    already count the new token."""
    _lib.oscar_decode_step(cache.dims, rot.struct, cache.struct(), k_new, v_new, q, ws.max_seq_len,
                           ws.buf, ws.nbytes, out, lse, stream, options)
