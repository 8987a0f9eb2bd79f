"""Shared pieces of the GPU parity tests: oracle-side inputs regenerated from
the seeded generator, and comparison bars.

Expected values always come from ``oracle/`` on inputs from ``synth``; no
value read back from the GPU is fed to the oracle.
"""
from __future__ import annotations

import numpy as np

from oracle import cpp as C
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


def oracle_request(model, layout, cal, q_bits_b, b: int, L: int, impl: str = "numpy"):
    """Oracle output [Hq][128] and lse [Hq] of request b at length L, from
    the numpy oracle or (impl "cpp") the plain C++ oracle."""
    k, v = request_tokens(model, layout, b, L)
    fn = C.request_attention if impl == "cpp" else O.request_attention
    return fn(q_bits_b, k, v, cal["r_k32"], cal["r_v32"], cal["clip_k"], cal["clip_v"], model.w.group_size,
              CODEBOOK_NAMES[model.w.codebook])


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


def assert_demoted_slot(page_block: np.ndarray, slot: int, k_bits: np.ndarray, v_bits: np.ndarray,
                        r_k32, r_v32, clip_k, clip_v, group: int, codebook: str, what: str = "") -> None:
    """One demoted history slot of a (page, KV head) block read back from the
    GPU against the oracle's demotion of the same bf16 token (k_bits,
    v_bits [128]).  Scale and zero are bit-exact; codes are equal except
    where (y - zero) / scale lies within 1e-5 (relative) of a level boundary,
    the tolerance of the acceptance bar for the rotation's last-bit
    rounding."""
    got = O.unpack_block(page_block, group)
    for which, bits, r, c, (gc, gs, gz) in (("k", k_bits, r_k32, clip_k, got[0:3]),
                                            ("v", v_bits, r_v32, clip_v, got[3:6])):
        y = O.clip(O.rotate(O.bf16_value(bits[None, :]), r), c)
        codes, s, z = O.quantize(y, group, codebook)
        assert np.array_equal(gs[slot], s[0]) and np.array_equal(gz[slot], z[0]), f"{what} {which} scale/zero"
        diff = gc[slot] != codes[0]
        if diff.any():
            sr = np.repeat(s[0], group).astype(np.float64)
            zr = np.repeat(z[0], group).astype(np.float64)
            t = (y[0].astype(np.float64) - zr) / np.where(sr == 0, 1, sr)
            if codebook == "uniform":
                near = np.abs(t - np.floor(t) - 0.5) <= 1e-5 * np.maximum(np.abs(t), 1)
            else:
                _, thr = O.lloyd_max_codebook()
                near = np.min(np.abs(t[:, None] - thr[None, :].astype(np.float64)), axis=1) <= \
                    1e-5 * np.maximum(np.abs(t), 1)
            assert not (diff & ~near).any(), f"{what} {which} codes differ away from a level boundary"
