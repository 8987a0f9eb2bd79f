"""Shared pieces of the GPU parity tests: oracle-side inputs regenerated from
the seeded generator, and comparison bars.

Expected values always come from ``oracle/`` on inputs from ``synth``; no
value read back from the GPU is fed to the oracle.
"""
from __future__ import annotations

import numpy as np

from oracle import oscar as O
from synth import gen

# Oracle names of the library's codebooks (Workload.codebook).
CODEBOOK_NAMES = {0: "uniform", 1: "lloyd-max"}

# Attention parity bar over the same dequantized cache (absolute max and
# relative L2 of the output).
ATOL = 2e-3
REL_L2 = 1e-3


def oracle_calibration(model):
    q, k, v = model.calibration()
    return O.calibrate(q, k, v, model.w.clip_pct)


def request_tokens(model, layout, b: int, L: int):
    """bf16 bits [L][Hkv][128] of the K and V tokens of request b (position
    order), regenerated on the host exactly as the GPU generator wrote them."""
    w = model.w
    k = np.zeros((L, w.num_kv_heads, 128), dtype=np.uint16)
    v = np.zeros_like(k)
    for j in range(w.num_kv_heads):
        for src, p0, n in layout.src_ranges(b, 0, L):
            k[p0:p0 + n, j] = gen.kv_tokens_bf16(w.seed, "k", src, j, p0, n, model.k_scale[j])
            v[p0:p0 + n, j] = gen.kv_tokens_bf16(w.seed, "v", src, j, p0, n, model.v_scale[j])
    return k, v


def oracle_request(model, layout, cal, q_bits_b, b: int, L: int, heads=None):
    """Oracle output [Hq][128] and lse [Hq] of request b at length L."""
    k, v = request_tokens(model, layout, b, L)
    return O.request_attention(q_bits_b, k, v, cal["r_k32"], cal["r_v32"], cal["clip_k"],
                               cal["clip_v"], model.w.group_size, CODEBOOK_NAMES[model.w.codebook])


def oracle_request_heads(model, layout, cal, q_bits_b, b: int, L: int, kv_heads):
    """Oracle output of the query groups of the listed KV heads of request b:
    {kv head: (out [g][128], lse [g])}."""
    w = model.w
    g = w.gqa
    res = {}
    for j in kv_heads:
        k = np.zeros((L, 1, 128), dtype=np.uint16)
        v = np.zeros_like(k)
        for src, p0, n in layout.src_ranges(b, 0, L):
            k[p0:p0 + n, 0] = gen.kv_tokens_bf16(w.seed, "k", src, j, p0, n, model.k_scale[j])
            v[p0:p0 + n, 0] = gen.kv_tokens_bf16(w.seed, "v", src, j, p0, n, model.v_scale[j])
        res[j] = O.request_attention(q_bits_b[j * g:(j + 1) * g], k, v, cal["r_k32"][j:j + 1],
                                     cal["r_v32"][j:j + 1], cal["clip_k"][j:j + 1],
                                     cal["clip_v"][j:j + 1], w.group_size, CODEBOOK_NAMES[w.codebook])
    return res


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = "", atol: float = ATOL,
                 rel_l2: float = REL_L2) -> None:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref).max()
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= atol and rel <= rel_l2, f"{what}: max-abs {err:.3e} rel-L2 {rel:.3e}"
