"""Synthetic workloads on the GPU: page tables and a filled cache.

Raw bf16 tokens come from the seeded generator (``synth``), on the GPU for
the large buffers; history pages are then written by the library's own bulk
demotion (``oscar_kv_fill_history``).  Host-side bookkeeping only.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from synth import configs, gen
from synth import gpu as synth_gpu

from . import _lib
from .kvcache import PagedKVCache, Rotation

BF16_TOKENS = _lib.SINK + _lib.RECENT


def hist_pages(L: int) -> int:
    return math.ceil(max(0, L - BF16_TOKENS) / _lib.PAGE)


class Layout:
    """Per-request lengths, shared-prefix sizes and the page table."""

    def __init__(self, w: configs.Workload, lens=None, extra_tokens: int = 0):
        self.w = w
        self.lens = np.array(lens if lens is not None else w.seq_lens, dtype=np.int64)
        B = w.batch
        assert self.lens.size == B
        now = [hist_pages(int(L)) for L in self.lens]
        alloc = [hist_pages(int(L) + extra_tokens) for L in self.lens]
        self.shared_pages = [n // 2 for n in now] if w.shared_prefix else [0] * B
        self.chain_len = max(self.shared_pages) if B else 0
        private = [a - s for a, s in zip(alloc, self.shared_pages)]
        total = self.chain_len + sum(private)
        self.n_pages = max(total, 1)
        ids = gen.permutation(w.seed, total) if (w.paged and total > 0) else np.arange(total, dtype=np.int32)
        self.max_pages = max(max(alloc) if B else 1, 1)
        pt = np.zeros((B, self.max_pages), dtype=np.int32)
        chain = ids[:self.chain_len]
        nxt = self.chain_len
        for b in range(B):
            sp = self.shared_pages[b]
            pt[b, :sp] = chain[:sp]
            pt[b, sp:alloc[b]] = ids[nxt:nxt + private[b]]
            nxt += private[b]
        self.page_table = pt
        self.prefix_len = [(_lib.SINK + _lib.PAGE * sp) if sp > 0 else 0 for sp in self.shared_pages]

    def src(self, b: int, pos: int) -> int:
        """Generator source id of position pos of request b."""
        return gen.SHARED_SRC if pos < self.prefix_len[b] else b

    def src_ranges(self, b: int, pos0: int, n: int):
        """Split [pos0, pos0+n) into (src, pos0, n) runs of one source."""
        cut = self.prefix_len[b]
        out = []
        if pos0 < cut:
            m = min(n, cut - pos0)
            out.append((gen.SHARED_SRC, pos0, m))
            pos0, n = pos0 + m, n - m
        if n > 0:
            out.append((b, pos0, n))
        return out


class SyntheticModel:
    """Model-level synthetic properties of a workload: query channel scales
    and the K/V outlier channels."""

    def __init__(self, w: configs.Workload):
        self.w = w
        self.sigma = gen.query_sigma(w.seed, w.num_q_heads, w.anisotropic_q)
        self.k_scale, self.v_scale = gen.outlier_scales(w.seed, w.num_kv_heads)

    def calibration(self):
        w = self.w
        return gen.calibration_tokens(w.seed + 1000, w.calib_tokens, w.num_q_heads, w.num_kv_heads,
                                      self.sigma, self.k_scale, self.v_scale)

    def queries(self, step: int, batch: int) -> np.ndarray:
        return gen.queries_bf16(self.w.seed, step, batch, self.w.num_q_heads, self.sigma)


def _bits_to_bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def queries_tensor(model: SyntheticModel, step: int, batch: int, device="cuda") -> torch.Tensor:
    return _bits_to_bf16_tensor(model.queries(step, batch), device)


def new_tokens_tensor(model: SyntheticModel, layout: Layout, step_lens, which: str,
                      device="cuda") -> torch.Tensor:
    """bf16 [B][Hkv][128] tokens at position L_b - 1 of each request."""
    w = model.w
    scale = model.k_scale if which == "k" else model.v_scale
    out = np.zeros((w.batch, w.num_kv_heads, 128), dtype=np.uint16)
    for b in range(w.batch):
        p = int(step_lens[b]) - 1
        src = layout.src(b, p)
        for j in range(w.num_kv_heads):
            out[b, j] = gen.kv_tokens_bf16(w.seed, which, src, j, p, 1, scale[j])[0]
    return _bits_to_bf16_tensor(out, device)


def build_cache(w: configs.Workload, layout: Layout, model: SyntheticModel, rot: Rotation,
                device: str = "cuda", chunk_tokens: int = 16384, stale_byte=None) -> PagedKVCache:
    """Allocate the cache and fill it to the layout's lengths: sink and recent
    from the GPU generator, history through the library's bulk demotion.
    With stale_byte set, every byte of the pages and of the sink/recent
    buffers holds that value before the fill, so the slots past each
    request's end keep it (0xFF: bf16 NaN scale/zero pairs, code 3)."""
    cache = PagedKVCache(w.num_q_heads, w.num_kv_heads, w.group_size, w.batch, layout.max_pages,
                         layout.n_pages, device, codebook=w.codebook)
    if stale_byte is not None:
        for t in (cache.pages, cache.sink_k, cache.sink_v, cache.recent_k, cache.recent_v):
            t.view(torch.uint8).fill_(stale_byte)
    cache.page_table.copy_(torch.from_numpy(layout.page_table))
    cache.seq_lens.copy_(torch.from_numpy(layout.lens.astype(np.int32)))
    stream = torch.cuda.current_stream().cuda_stream
    hkv = w.num_kv_heads
    ks = torch.from_numpy(model.k_scale).to(device)
    vs = torch.from_numpy(model.v_scale).to(device)
    seed = w.seed

    def fill(dst: torch.Tensor, elem_off: int, b: int, pos0: int, n: int, stride_t: int,
             stride_h: int, which: str):
        scale = ks if which == "k" else vs
        for src, p0, m in layout.src_ranges(b, pos0, n):
            addr = dst.data_ptr() + 2 * (elem_off + (p0 - pos0) * stride_t)
            synth_gpu.fill_kv(addr, m, hkv, stride_t, stride_h, seed, which, src, p0, scale, stream)

    per_req_sink = hkv * _lib.SINK * 128
    per_req_recent = hkv * _lib.RECENT * 128
    for b in range(w.batch):
        L = int(layout.lens[b])
        n_s = min(L, _lib.SINK)
        n_r = min(max(L - _lib.SINK, 0), _lib.RECENT)
        for which, sink, recent in (("k", cache.sink_k, cache.recent_k), ("v", cache.sink_v, cache.recent_v)):
            if n_s:
                fill(sink, b * per_req_sink, b, 0, n_s, 128, _lib.SINK * 128, which)
            p = L - n_r
            while p < L:
                slot = (p - _lib.SINK) % _lib.RECENT
                m = min(L - p, _lib.RECENT - slot)
                fill(recent, b * per_req_recent + slot * 128, b, p, m, 128, _lib.RECENT * 128, which)
                p += m
    # history: the shared chain once, then each request's private part
    stage_k = torch.empty((chunk_tokens, hkv, 128), dtype=torch.bfloat16, device=device)
    stage_v = torch.empty_like(stage_k)
    cs = cache.struct()

    def fill_hist(b: int, j0: int, j1: int):
        j = j0
        while j < j1:
            n = min(chunk_tokens, j1 - j)
            fill(stage_k, 0, b, _lib.SINK + j, n, hkv * 128, 128, "k")
            fill(stage_v, 0, b, _lib.SINK + j, n, hkv * 128, 128, "v")
            _lib.oscar_kv_fill_history(cache.dims, rot.struct, cs, b, j, n, stage_k, stage_v, stream)
            j += n

    if layout.chain_len > 0:
        owner = int(np.argmax(layout.shared_pages))
        fill_hist(owner, 0, _lib.PAGE * layout.shared_pages[owner])
    for b in range(w.batch):
        n_h = max(0, int(layout.lens[b]) - BF16_TOKENS)
        fill_hist(b, _lib.PAGE * layout.shared_pages[b], n_h)
    torch.cuda.current_stream().synchronize()
    return cache


def build_bf16_cache(w: configs.Workload, layout: Layout, device: str = "cuda", chunk_tokens: int = 16384,
                     extra_tokens: int = 0):
    """The all-bf16 baseline cache holding the same tokens as build_cache
    (every position of every request in bf16 pages, filled from the GPU
    generator through oscar_bf16_fill).  Pages are a seeded permutation."""
    from .kvcache import Bf16PagedCache
    B, hkv = w.batch, w.num_kv_heads
    lens = layout.lens
    need = [-(-(int(L) + extra_tokens) // _lib.PAGE) for L in lens]
    total = max(sum(need), 1)
    ids = gen.permutation(w.seed + 7, total) if w.paged else np.arange(total, dtype=np.int32)
    max_pages = max(max(need), 1)
    pt = np.zeros((B, max_pages), dtype=np.int32)
    nxt = 0
    for b in range(B):
        pt[b, :need[b]] = ids[nxt:nxt + need[b]]
        nxt += need[b]
    cache = Bf16PagedCache(w.num_q_heads, hkv, B, max_pages, total, device)
    cache.page_table.copy_(torch.from_numpy(pt))
    cache.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    model = SyntheticModel(w)
    ks = torch.from_numpy(model.k_scale).to(device)
    vs = torch.from_numpy(model.v_scale).to(device)
    stream = torch.cuda.current_stream().cuda_stream
    stage_k = torch.empty((chunk_tokens, hkv, 128), dtype=torch.bfloat16, device=device)
    stage_v = torch.empty_like(stage_k)
    cs = cache.struct()
    for b in range(B):
        L = int(lens[b])
        p = 0
        while p < L:
            n = min(chunk_tokens, L - p)
            for dst, which, scale in ((stage_k, "k", ks), (stage_v, "v", vs)):
                for src, p0, m in layout.src_ranges(b, p, n):
                    synth_gpu.fill_kv(dst.data_ptr() + 2 * (p0 - p) * hkv * 128, m, hkv, hkv * 128, 128,
                                      w.seed, which, src, p0, scale, stream)
            _lib.oscar_bf16_fill(cache.dims, cs, b, p, n, stage_k, stage_v, stream)
            p += n
    torch.cuda.current_stream().synchronize()
    return cache
