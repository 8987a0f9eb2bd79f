"""Pins of the plain C++ oracle (oracle/oscar_ref.cpp) on the CPU.

The C++ oracle is a second, independent writing of the decode path's
arithmetic (demotion, dequantization, one softmax over sink + history +
recent).  It is pinned here against the numpy oracle, which the pins in
test_oracle_pins.py tie to the pages and to the mathematics: codes, scales
and zero points bit-exact, attention outputs to 1e-12; against explicit
loops where a request has no history; and against the published levels of
the four-level Gaussian Lloyd-Max quantizer.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import cpp as C
from oracle import oscar as O
from synth import gen


def rng(seed):
    return np.random.default_rng(seed)


def _rotations(r, n):
    out = []
    for _ in range(n):
        _, u = O.eig_descending(np.cov(r.standard_normal((300, 128)).T))
        out.append(O.composite_rotation(u).astype(np.float32))
    return np.stack(out)


def _tokens(r, shape, outliers=True):
    x = r.standard_normal(shape)
    if outliers:
        x[..., 5] *= 20.0
        x[..., 77] *= 8.0
    return gen.bf16_bits(x.astype(np.float32))


def test_lloyd_max_levels():
    """Same codebook as the numpy oracle, and the published four-level
    normal quantizer (levels +-0.4528, +-1.510; thresholds 0, +-0.9816)."""
    lev, thr = C.lloyd_max()
    ol, ot = O.lloyd_max_gaussian()
    assert np.abs(lev - ol).max() < 1e-15
    assert np.abs(thr - ot).max() < 1e-15
    assert np.allclose(lev, [-1.5104, -0.4528, 0.4528, 1.5104], atol=1e-4)
    assert np.allclose(thr, [-0.9816, 0.0, 0.9816], atol=1e-4)


@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("codebook", ["uniform", "lloyd-max"])
def test_demote_bit_exact_with_numpy_oracle(group, codebook):
    r = rng(7 + group)
    n = 1500
    x = _tokens(r, (n, 128))
    x[3] = 0                                   # all-zero token: scale 0, codes 0
    x[4] = gen.bf16_bits(np.full(128, 1.5, np.float32))
    rot = _rotations(r, 1)[0]
    clip = np.full(128, 3.0, np.float32)
    clip[::7] = 0.25                           # clipped channels
    ref = O.demote(x, rot, clip, group, codebook)
    got = C.demote(x, rot, clip, group, codebook)
    for a, b, name in zip(got, ref, ("codes", "scale", "zero")):
        assert a.dtype == b.dtype and a.shape == b.shape, name
        assert np.array_equal(a, b), f"{name}: {int((a != b).sum())} differ"
    # Identity rotation and a constant token: every group has scale 0.
    eye = np.eye(128, dtype=np.float32)
    const = gen.bf16_bits(np.full((2, 128), -0.75, np.float32))
    codes, s, z = C.demote(const, eye, np.full(128, 10.0, np.float32), group, codebook)
    assert not codes.any() and not s.any() and np.all(z == -0.75)


def _case(L, hq, hkv, seed):
    r = rng(seed)
    k = _tokens(r, (L, hkv, 128))
    v = _tokens(r, (L, hkv, 128), outliers=False)
    q = gen.bf16_bits(r.standard_normal((hq, 128)).astype(np.float32))
    rots = _rotations(r, 2 * hkv)
    ck = np.full((hkv, 128), 4.0, np.float32)
    cv = np.full((hkv, 128), 2.5, np.float32)
    return q, k, v, rots[:hkv], rots[hkv:], ck, cv


@pytest.mark.parametrize("L", [1, 63, 64, 65, 320, 321, 333, 700, 2100])
@pytest.mark.parametrize("codebook", ["uniform", "lloyd-max"])
def test_request_attention_matches_numpy_oracle(L, codebook):
    q, k, v, rk, rv, ck, cv = _case(L, 8, 2, 1000 + L)
    for group in (32, 128):
        ro, rl = O.request_attention(q, k, v, rk, rv, ck, cv, group, codebook)
        go, gl = C.request_attention(q, k, v, rk, rv, ck, cv, group, codebook)
        assert np.abs(go - ro).max() < 1e-12 * max(1.0, np.abs(ro).max())
        assert np.abs(gl - rl).max() < 1e-12 * max(1.0, np.abs(rl).max())


@pytest.mark.parametrize("L", [1, 5, 64, 300, 320])
def test_no_history_is_plain_attention(L):
    """With L <= 320 every token stays bf16: the output is softmax attention
    of the bf16 values, written out with explicit loops (fsum)."""
    q, k, v, rk, rv, ck, cv = _case(L, 2, 1, 50 + L)
    out, lse = C.request_attention(q, k, v, rk, rv, ck, cv, 64)
    qv, kv, vv = O.bf16_value(q), O.bf16_value(k[:, 0]), O.bf16_value(v[:, 0])
    for h in range(2):
        sc = [math.fsum(qv[h, c] * kv[t, c] for c in range(128)) / math.sqrt(128) for t in range(L)]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        tot = math.fsum(w)
        ref = np.array([math.fsum(w[t] * vv[t, c] for t in range(L)) / tot for c in range(128)])
        assert np.abs(out[h] - ref).max() < 1e-12
        assert abs(lse[h] - (m + math.log(tot))) < 1e-12


def test_threads_give_identical_results():
    """Pairs are independent: any number of OpenMP threads gives the same bits."""
    q, k, v, rk, rv, ck, cv = _case(900, 16, 4, 77)
    one = C.request_attention(q, k, v, rk, rv, ck, cv, 64, threads=1)
    many = C.request_attention(q, k, v, rk, rv, ck, cv, 64, threads=4)
    assert np.array_equal(one[0], many[0]) and np.array_equal(one[1], many[1])


def test_rejects_bad_arguments():
    q, k, v, rk, rv, ck, cv = _case(10, 2, 1, 5)
    with pytest.raises(ValueError):
        C.request_attention(q, k, v, rk, rv, ck, cv, 48)
    with pytest.raises(ValueError):
        C.demote(k[:, 0], rk[0], ck[0], 100)
    assert C.attend_pairs([], 4, 64) == []
