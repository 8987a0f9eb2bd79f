"""Workload shapes of the synthetic caches (sizes and seeds only).

Shapes follow the workloads the OSCAR pages describe: query/KV head
counts of the Qwen3 models they evaluate, 100K and 128K contexts, batch 1
and 32, paged caches with 64-token pages, and a shared prefix.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    group_size: int              # quantization group G (channels)
    batch: int
    seq_lens: tuple              # L per request at attention time (incl. current token)
    paged: bool = True           # random page-table permutation; else identity
    shared_prefix: bool = False  # first floor(pages/2) history pages shared across requests
    anisotropic_q: bool = True
    calib_tokens: int = 2048
    clip_pct: float = 99.9
    steps: int = 1
    extra: dict = field(default_factory=dict)
    codebook: int = 0            # history codebook: 0 uniform (min/max), 1 Lloyd-Max

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def tiny() -> Workload:
    """1 KV head, 1 query head, batch 1, context 1024 = 64 | 704 | 256, G = 32."""
    return Workload("tiny", 0, 1, 1, 32, 1, (1024,), paged=False, anisotropic_q=False)


def qwen3_8b_b1(steps: int = 100) -> Workload:
    """32 q / 8 kv heads, batch 1, 100K context, contiguous history, G = 128."""
    return Workload("qwen3-8b-b1-100k", 1, 32, 8, 128, 1, (100_000,), paged=False, steps=steps)


def qwen3_8b_b32(group_size: int = 128) -> Workload:
    """32 q / 8 kv heads, batch 32, every request at 100K, paged (64), G = 128 or 64."""
    return Workload(f"qwen3-8b-b32-100k-g{group_size}", 2, 32, 8, group_size, 32,
                    (100_000,) * 32, paged=True)


def qwen3_4b_b16() -> Workload:
    """32 q / 8 kv heads, batch 16, 128K context, paged (64), G = 128."""
    return Workload("qwen3-4b-b16-128k", 3, 32, 8, 128, 16, (131_072,) * 16, paged=True)


def qwen3_32b_ragged(seq_lens: tuple) -> Workload:
    """64 q / 8 kv heads (GQA 8), batch 32, ragged 4K..128K, shared prefix, G = 128."""
    return Workload("qwen3-32b-b32-ragged", 4, 64, 8, 128, 32, tuple(seq_lens),
                    paged=True, shared_prefix=True, steps=200)


PAGE = 64
SINK = 64
RECENT = 256
HEAD_DIM = 128
