"""Pins of the CPU oracle against what the OSCAR pages and mathematics fix.

Each test checks an oracle function against something other than itself:
a closed form, an invariant, a special case that reduces to a textbook or
library routine, brute force on tiny inputs, or the figures the pages print
(tests/golden/page_figures.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oscar as O
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------- P1
def test_hadamard_closed_form_and_fwht():
    h = O.hadamard(128)
    for i in range(128):
        for k in range(128):
            assert h[i, k] == (-1) ** bin(i & k).count("1") / math.sqrt(128)
    assert np.array_equal(h, h.T)
    assert np.abs(h @ h - np.eye(128)).max() < 1e-14
    # fast Walsh-Hadamard butterflies (natural order) equal the matrix product
    x = rng(1).standard_normal((5, 128))
    y = x.copy()
    span = 1
    while span < 128:
        for start in range(0, 128, 2 * span):
            a = y[:, start:start + span].copy()
            b = y[:, start + span:start + 2 * span].copy()
            y[:, start:start + span] = a + b
            y[:, start + span:start + 2 * span] = a - b
        span *= 2
    assert np.abs(y / math.sqrt(128) - x @ h).max() < 1e-12


# --------------------------------------------------------------------- P4
def test_bit_reversal():
    assert O.bit_reverse(1) == 64 and O.bit_reverse(3) == 96 and O.bit_reverse(127) == 127
    assert all(O.bit_reverse(O.bit_reverse(i)) == i for i in range(128))
    p = O.bit_reversal_matrix(128)
    assert np.array_equal(p, p.T) and np.array_equal(p @ p, np.eye(128))
    x = np.arange(128.0)
    assert np.array_equal(x @ p, np.array([O.bit_reverse(k) for k in range(128)], dtype=float))
    # each group of 32 consecutive stored channels takes one channel from
    # every block of 4 consecutive source channels (interleaving across groups)
    src = np.array([O.bit_reverse(k) for k in range(128)])
    for g0 in range(0, 128, 32):
        assert sorted(src[g0:g0 + 32] // 4) == list(range(32))


# --------------------------------------------------------------------- P2/P3
def test_eig_diagonal_gives_signed_permutation():
    d = np.array([3.0, 7.0, 1.0, 5.0] + list(np.linspace(0.01, 0.5, 124)))
    lam, u = O.eig_descending(np.diag(d))
    assert np.allclose(lam, np.sort(d)[::-1], rtol=1e-12, atol=0)
    assert np.array_equal(np.abs(u).round(12), np.abs(u).round(12).astype(bool).astype(float))
    assert np.array_equal(np.argmax(np.abs(u), axis=0), np.argsort(-d, kind="stable"))
    assert (u[np.argmax(np.abs(u), axis=0), range(128)] > 0).all()


def test_eig_two_by_two_closed_form():
    a, b = 2.0, 0.75
    lam, u = O.eig_descending(np.array([[a, b], [b, a]]))
    assert np.allclose(lam, [a + b, a - b], atol=1e-15)
    s = 1 / math.sqrt(2)
    assert np.allclose(u[:, 0], [s, s], atol=1e-15)
    assert np.allclose(np.abs(u[:, 1]), [s, s], atol=1e-15)
    assert u[0, 1] > 0  # tie on magnitude: lowest index made positive


def test_eig_reconstruction_and_order():
    x = rng(2).standard_normal((300, 128))
    c = x.T @ x / 300
    lam, u = O.eig_descending(c)
    assert np.all(np.diff(lam) <= 0)
    assert np.abs(u.T @ u - np.eye(128)).max() < 1e-12
    assert np.abs(u @ np.diag(lam) @ u.T - c).max() < 1e-12 * np.abs(c).max() * 10


def test_rotation_uniform_diagonal_closed_form():
    """diag(R^T C R) = tr(C)/128 for R = U H P, U the eigenvectors of C."""
    x = rng(3).standard_normal((400, 128)) * np.exp(rng(4).standard_normal(128))
    c = x.T @ x / 400
    _, u = O.eig_descending(c)
    r = O.composite_rotation(u)
    d = np.diag(r.T @ c @ r)
    assert np.abs(d - np.trace(c) / 128).max() < 1e-10 * np.trace(c)
    # a wrong factor order (H U P) breaks the uniformity
    wrong = O.hadamard() @ u @ O.bit_reversal_matrix()
    assert np.abs(np.diag(wrong.T @ c @ wrong) - np.trace(c) / 128).max() > 1e-3 * np.trace(c)


# ------------------------------------------------------------ covariances
def test_query_covariance_reduces_to_library_cov():
    q = rng(5).standard_normal((64, 4, 128)) + 0.3
    rows = q.reshape(-1, 128)
    mu = rows.mean(axis=0)
    ref = np.cov(rows.T, bias=True) + np.outer(mu, mu)
    assert np.abs(O.query_covariance(q) - ref).max() < 1e-12


def test_causal_attention_special_cases():
    r = rng(6)
    n = 9
    k = r.standard_normal((n, 128))
    v = r.standard_normal((n, 128))
    # zero queries: uniform over visible keys -> cumulative means
    o = O.causal_attention_outputs(np.zeros((n, 128)), k, v)
    cum = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.abs(o - cum).max() < 1e-13
    # brute force, two-pass softmax with explicit loops
    q = r.standard_normal((n, 128))
    o = O.causal_attention_outputs(q, k, v)
    for i in range(n):
        sc = [sum(q[i, c] * k[t, c] for c in range(128)) / math.sqrt(128) for t in range(i + 1)]
        m = max(sc)
        w = [math.exp(s - m) for s in sc]
        tot = sum(w)
        for c in range(0, 128, 17):
            ref = sum(w[t] * v[t, c] for t in range(i + 1)) / tot
            assert abs(o[i, c] - ref) < 1e-12


def test_score_weighted_value_covariance_zero_query_closed_form():
    r = rng(7)
    n, g = 12, 2
    k = r.standard_normal((n, 128))
    v = r.standard_normal((n, 128))
    cum = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    ref = cum.T @ cum / n
    got = O.score_weighted_value_covariance(np.zeros((n, g, 128)), k, v)
    assert np.abs(got - ref).max() < 1e-12
    # pooling over the group is the mean of the per-head covariances
    q = r.standard_normal((n, g, 128))
    per = [O.score_weighted_value_covariance(q[:, h:h + 1], k, v) for h in range(g)]
    assert np.abs(O.score_weighted_value_covariance(q, k, v) - sum(per) / g).max() < 1e-12


def test_clip_threshold_percentile_closed_form():
    # |y| takes the values 0..2047 in every channel; the 99.9th percentile with
    # linear interpolation sits at rank 0.999 * 2047 = 2044.953
    x = np.tile(np.arange(2048.0)[:, None], (1, 128))
    x[1::2] *= -1
    c = O.clip_thresholds(x, np.eye(128), 99.9)
    assert np.allclose(c, 2044.953, rtol=0, atol=1e-3)
    assert c.dtype == np.float32


# --------------------------------------------------------------------- P7
@pytest.fixture(scope="module")
def tiny_calibration():
    from synth import configs
    w = configs.tiny()
    sigma = gen.query_sigma(w.seed, w.num_q_heads, w.anisotropic_q)
    ks, vs = gen.outlier_scales(w.seed, w.num_kv_heads)
    q, k, v = gen.calibration_tokens(w.seed + 1000, w.calib_tokens, w.num_q_heads,
                                     w.num_kv_heads, sigma, ks, vs)
    return O.calibrate(q, k, v, w.clip_pct), (q, k, v)


def test_rotations_orthogonal(tiny_calibration):
    cal, _ = tiny_calibration
    for r in (cal["r_k"][0], cal["r_v"][0]):
        assert np.abs(r.T @ r - np.eye(128)).max() <= 1e-10
    # float32 copies are orthogonal to float32 precision
    for r in (cal["r_k32"][0], cal["r_v32"][0]):
        r = r.astype(np.float64)
        assert np.abs(r.T @ r - np.eye(128)).max() <= 1e-6


def _brute_value_outputs(q, k, v):
    """Causal softmax attention outputs, one query row at a time (explicit
    two-pass softmax), for the calibration-wiring pin."""
    n = q.shape[0]
    out = np.zeros((n, 128))
    for i in range(n):
        sc = np.array([float(np.dot(q[i], k[t])) for t in range(i + 1)]) / math.sqrt(128)
        w = np.exp(sc - sc.max())
        out[i] = (w[:, None] * v[:i + 1]).sum(axis=0) / w.sum()
    return out


def _wiring_inputs():
    """A small GQA-2 calibration set whose query covariance and score-weighted
    value covariance differ strongly: queries with log-normal channel scales
    and a mean, values with two x10 channels, keys correlated with queries."""
    r = rng(41)
    n, g, hkv = 96, 2, 2
    qs = np.exp(r.standard_normal(128))
    q = r.standard_normal((n, g * hkv, 128)) * qs + 0.2 * qs
    k = r.standard_normal((n, hkv, 128)) + 0.3 * q[:, ::g, :] / qs.max()
    v = r.standard_normal((n, hkv, 128))
    v[:, :, 5] *= 10
    v[:, :, 77] *= 10
    return q, k, v, g


def _wiring_failures(cal, q, k, v, g):
    """What P2 and the clip definition fix about calibrate()'s outputs, per KV
    head j, with C_Q and C_S recomputed here from their definitions:
    diag(R_K^T C_Q R_K) and diag(R_V^T C_S R_V) are uniform at tr/128, the
    crossed pairings are not, and clip_k / clip_v are the 99.9th percentiles
    of |k R_K| / |v R_V| per channel."""
    bad = []
    for j in range(k.shape[1]):
        rows = q[:, j * g:(j + 1) * g, :].reshape(-1, 128)
        c_q = rows.T @ rows / rows.shape[0]
        outs = np.concatenate([_brute_value_outputs(q[:, h, :], k[:, j], v[:, j])
                               for h in range(j * g, (j + 1) * g)])
        c_s = outs.T @ outs / outs.shape[0]
        rk, rv = cal["r_k"][j], cal["r_v"][j]

        def spread(r, c):
            return np.abs(np.diag(r.T @ c @ r) - np.trace(c) / 128).max() / np.trace(c)

        if spread(rk, c_q) > 1e-10:
            bad.append(f"kvh {j}: diag(R_K^T C_Q R_K) not uniform")
        if spread(rv, c_s) > 1e-10:
            bad.append(f"kvh {j}: diag(R_V^T C_S R_V) not uniform")
        if spread(rk, c_s) < 1e-3 or spread(rv, c_q) < 1e-3:
            bad.append(f"kvh {j}: a crossed pairing is uniform too (inputs do not separate them)")
        ck = np.percentile(np.abs(k[:, j] @ rk), 99.9, axis=0).astype(np.float32)
        cv = np.percentile(np.abs(v[:, j] @ rv), 99.9, axis=0).astype(np.float32)
        if not np.array_equal(cal["clip_k"][j], ck):
            bad.append(f"kvh {j}: clip_k is not the p99.9 of |k R_K|")
        if not np.array_equal(cal["clip_v"][j], cv):
            bad.append(f"kvh {j}: clip_v is not the p99.9 of |v R_V|")
    return bad


def test_calibrate_pairs_each_rotation_with_its_covariance():
    """P2 on calibrate() as a whole ([A] section "OSCAR 的不同之处": R_K from
    the eigenvectors of C_Q, R_V from those of C_S = V^T S^T S V / N), GQA 2,
    and the clip thresholds from the matching rotation."""
    q, k, v, g = _wiring_inputs()
    cal = O.calibrate(q, k, v, 99.9)
    assert _wiring_failures(cal, q, k, v, g) == []


def test_calibrate_wiring_pin_catches_planted_mistakes():
    """Copies of calibrate_head with one plausible mistake each fail the
    wiring pin: U_Q and U_S swapped, clip_v taken from the keys, C_S built
    from pre-softmax scores, and the query group of the wrong KV head."""
    q, k, v, g = _wiring_inputs()

    def variant(mistake):
        heads = []
        for j in range(k.shape[1]):
            jq = (j + 1) % k.shape[1] if mistake == "group" else j
            qj, kj, vj = q[:, jq * g:(jq + 1) * g, :], k[:, j, :], v[:, j, :]
            _, u_q = O.eig_descending(O.query_covariance(qj))
            if mistake == "scores":
                s = np.concatenate([np.tril(qj[:, h] @ kj.T / math.sqrt(128)) @ vj for h in range(g)])
                c_s = s.T @ s / s.shape[0]
            else:
                c_s = O.score_weighted_value_covariance(qj, kj, vj)
            _, u_s = O.eig_descending(c_s)
            if mistake == "swap":
                u_q, u_s = u_s, u_q
            r_k, r_v = O.composite_rotation(u_q), O.composite_rotation(u_s)
            clip_v = O.clip_thresholds(kj if mistake == "clip" else vj, r_v, 99.9)
            heads.append({"r_k": r_k, "r_v": r_v, "clip_k": O.clip_thresholds(kj, r_k, 99.9),
                          "clip_v": clip_v})
        return {key: np.stack([h[key] for h in heads]) for key in heads[0]}

    for mistake in ("swap", "clip", "scores", "group"):
        assert _wiring_failures(variant(mistake), q, k, v, g), mistake
    assert _wiring_failures(variant("none"), q, k, v, g) == []


def test_calibration_spreads_outlier_channels(tiny_calibration):
    cal, (_, k, _) = tiny_calibration
    raw_max = np.percentile(np.abs(k[:, 0]), 99.9, axis=0)
    clip_k = cal["clip_k"][0]
    # raw keys have 4 channels at x20; after rotation the per-channel spread
    # is far more even (Hadamard and bit reversal equalise energy)
    assert raw_max.max() / np.median(raw_max) > 10
    assert clip_k.max() / np.median(clip_k) < 4


# --------------------------------------------------------------------- P5
def test_pack_unpack_roundtrip_and_byte_values():
    r = rng(8)
    for group in (32, 64, 128):
        ng = 128 // group
        ck = r.integers(0, 4, (64, 128)).astype(np.uint8)
        cv = r.integers(0, 4, (64, 128)).astype(np.uint8)
        sk = O.bf16_round(r.standard_normal((64, ng)).astype(np.float32))
        zk = O.bf16_round(r.standard_normal((64, ng)).astype(np.float32))
        sv = O.bf16_round(r.standard_normal((64, ng)).astype(np.float32))
        zv = O.bf16_round(r.standard_normal((64, ng)).astype(np.float32))
        blk = O.pack_block(ck, sk, zk, cv, sv, zv, group)
        assert blk.size == O.block_bytes(group)
        back = O.unpack_block(blk, group)
        for a, b in zip(back, (ck, sk, zk, cv, sv, zv)):
            assert np.array_equal(a, b)


def test_pack_byte_is_four_codes_lsb_first_all_values():
    """Every byte value 0..255 occurs, and each byte equals sum c_i 4^i of the
    four codes it holds (four consecutive channels of one token for K, four
    consecutive tokens of one channel for V) with its top bit flipped (the
    fourth code stored XOR 2)."""
    ck = np.zeros((64, 128), dtype=np.uint8)
    cv = np.zeros((64, 128), dtype=np.uint8)
    for t in range(64):
        for m in range(32):
            b = (t * 32 + m) % 256
            for i in range(4):
                ck[t, 4 * m + i] = (b >> (2 * i)) & 3
    for c in range(128):
        for m in range(16):
            b = (c * 16 + m * 7) % 256
            for i in range(4):
                cv[4 * m + i, c] = (b >> (2 * i)) & 3
    ng = 1
    z = np.zeros((64, ng), dtype=np.float32)
    blk = O.pack_block(ck, z, z, cv, z, z, 128)
    seen = set()
    for t in range(64):
        for d in range(8):
            word_off = 4 * (d * 64 + O.qk_order(t))
            for j in range(4):
                byte = int(blk[word_off + j])
                m = 4 * d + j
                assert byte == sum(int(ck[t, 4 * m + i]) << (2 * i) for i in range(4)) ^ 0x80
                seen.add(byte)
    assert seen == set(range(256))
    seen = set()
    for c in range(128):
        for w in range(4):
            word_off = 2048 + 4 * ((c // 64) * 256 + (w * 16 + c % 16) * 4 + (c // 16) % 4)
            for j in range(4):
                byte = int(blk[word_off + j])
                tok0 = 16 * w + 4 * j
                assert byte == sum(int(cv[tok0 + i, c]) << (2 * i) for i in range(4)) ^ 0x80
                seen.add(byte)
    assert seen == set(range(256))


def test_layout_maps_are_bijections():
    assert sorted(O.qk_order(t) for t in range(64)) == list(range(64))
    vmap = sorted((c // 64) * 256 + (w * 16 + c % 16) * 4 + (c // 16) % 4
                  for c in range(128) for w in range(4))
    assert vmap == list(range(512))


# --------------------------------------------------------------------- P6
def test_bf16_round_matches_torch():
    x = np.concatenate([rng(9).standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.5, 0.0, 3.0], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.bf16_round(x), ref)


def _levels_nearest(y, s, z):
    """Brute force: index of the nearest of the four levels z + k s (float64)."""
    lv = z[..., None].astype(np.float64) + np.arange(4) * s[..., None].astype(np.float64)
    return np.argmin(np.abs(y[..., None].astype(np.float64) - lv), axis=-1)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_quantizer_invariants_and_brute_force(group):
    r = rng(10 + group)
    y = (r.standard_normal((500, 128)) * np.exp(r.standard_normal(128))).astype(np.float32)
    codes, s, z = O.quantize_groups(y, group)
    ng = 128 // group
    assert codes.dtype == np.uint8 and codes.max() <= 3
    assert np.array_equal(O.bf16_round(s), s) and np.array_equal(O.bf16_round(z), z)
    yg = y.reshape(500, ng, group)
    assert np.array_equal(z, O.bf16_round(yg.min(axis=2)))
    yhat = O.dequantize(codes, s, z, group).reshape(500, ng, group)
    k = codes.reshape(500, ng, group).astype(np.float64)
    assert np.array_equal(yhat, (k * s[..., None] + z[..., None]).astype(np.float32))
    # error bound: half a step plus bf16 rounding of s and z
    err = np.abs(yhat.astype(np.float64) - yg)
    bound = s[..., None] / 2 + 2 ** -7 * (3 * s[..., None] + np.abs(yg.min(axis=2))[..., None])
    assert (err <= bound).all()
    # nearest level (brute force) except within 1e-5 of a decision boundary
    near = _levels_nearest(yg, s[..., None] * np.ones_like(yg), z[..., None] * np.ones_like(yg))
    t = (yg.astype(np.float64) - z[..., None]) / s[..., None]
    ambiguous = np.abs(t - np.floor(t) - 0.5) < 1e-5
    mismatch = (near != codes.reshape(500, ng, group)) & ~ambiguous
    assert not mismatch.any()
    # min and max land on the extreme levels
    assert (codes.reshape(500, ng, group).min(axis=2) == 0).all()
    assert (codes.reshape(500, ng, group).max(axis=2) == 3).all()


def test_quantizer_constant_group_and_permutation():
    y = np.full((3, 128), 1.7, dtype=np.float32)
    codes, s, z = O.quantize_groups(y, 64)
    assert (codes == 0).all() and (s == 0).all()
    assert np.array_equal(O.dequantize(codes, s, z, 64), np.broadcast_to(O.bf16_round(y[:, :1]), y.shape))
    # at G = 128 a channel permutation permutes the codes
    y = rng(11).standard_normal((50, 128)).astype(np.float32)
    perm = np.array([O.bit_reverse(i) for i in range(128)])
    c1, s1, z1 = O.quantize_groups(y, 128)
    c2, s2, z2 = O.quantize_groups(y[:, perm], 128)
    assert np.array_equal(c1[:, perm], c2) and np.array_equal(s1, s2) and np.array_equal(z1, z2)


def test_clip_then_quantize_respects_thresholds():
    y = (rng(12).standard_normal((40, 128)) * 5).astype(np.float32)
    c = np.full(128, 2.0, dtype=np.float32)
    yc = O.clip(y, c)
    assert yc.max() <= 2.0 and yc.min() >= -2.0
    assert np.array_equal(yc[np.abs(y) <= 2.0], y[np.abs(y) <= 2.0])


def test_rotate_is_single_rounding_of_exact_sum():
    r = rng(13)
    x = O.bf16_round(r.standard_normal((4, 128)).astype(np.float32))
    rot = r.standard_normal((128, 128)).astype(np.float32)
    y = O.rotate(x, rot)
    exact = [[math.fsum(float(x[i, j]) * float(rot[j, k]) for j in range(128)) for k in range(0, 128, 31)]
             for i in range(4)]
    assert np.array_equal(y[:, ::31], np.array(exact, dtype=np.float32))


# --------------------------------------------------------------------- P8
def test_rotation_without_quantization_is_invariant():
    r = rng(14)
    g, n_b, n_h = 4, 40, 200
    q_bits = gen.bf16_bits(r.standard_normal((g, 128)).astype(np.float32) * 2)
    kb = gen.bf16_bits(r.standard_normal((n_b, 128)).astype(np.float32))
    vb = gen.bf16_bits(r.standard_normal((n_b, 128)).astype(np.float32))
    kh = r.standard_normal((n_h, 128))
    vh = r.standard_normal((n_h, 128))
    _, u = O.eig_descending(np.cov(r.standard_normal((500, 128)).T))
    rk = O.composite_rotation(u)
    _, u2 = O.eig_descending(np.cov(r.standard_normal((500, 128)).T))
    rv = O.composite_rotation(u2)
    out, lse = O.attend(q_bits, kb, vb, kh @ rk, vh @ rv, rk, rv)
    q = O.bf16_value(q_bits)
    ref, ref_lse = O.partial_attend(q, np.concatenate([O.bf16_value(kb), kh]),
                                    np.concatenate([O.bf16_value(vb), vh]))
    assert np.abs(out - ref).max() < 1e-12
    assert np.abs(lse - ref_lse).max() < 1e-12


# --------------------------------------------------------------------- P9
def test_logit_error_identity():
    """||Q K^T - Q Khat^T||_F^2 = tr((K - Khat) Q^T Q (K - Khat)^T)."""
    r = rng(15)
    q = r.standard_normal((64, 128)) * np.exp(r.standard_normal(128))
    k = r.standard_normal((300, 128))
    k[:, [3, 50]] *= 20
    _, u = O.eig_descending(O.query_covariance(q[:, None, :]))
    rk = O.composite_rotation(u)
    rk32 = rk.astype(np.float32)
    clipv = np.percentile(np.abs(k @ rk), 99.9, axis=0).astype(np.float32)
    codes, s, z = O.quantize_groups(O.clip(O.rotate(k, rk32), clipv), 128)
    khat = O.dequantize(codes, s, z, 128).astype(np.float64) @ rk32.astype(np.float64).T
    lhs = np.linalg.norm(q @ k.T - q @ khat.T, "fro") ** 2
    dk = k - khat
    rhs = np.trace(dk @ q.T @ q @ dk.T)
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs)


# -------------------------------------------------------------------- P10
def _brute_dequant(codes, s, z, group, codebook):
    """One token's dequantized values, element by element."""
    lev = O.lloyd_max_codebook()[0]
    out = np.zeros(128)
    for c in range(128):
        gi = c // group
        k = int(codes[0, c])
        out[c] = (float(z[0, gi]) + float(s[0, gi]) * float(lev[k])) if codebook == "lloyd-max" \
            else float(np.float32(np.float32(k) * s[0, gi] + z[0, gi]))
    return out


def _brute_request(q_bits, k_bits, v_bits, rk, rv, ck, cv, group, codebook="uniform"):
    """Two-pass softmax with explicit loops over tokens; history keys and values
    are rotated back to the model domain (k_hat R^T, v_hat R^T) instead of
    rotating the query and the output."""
    L = k_bits.shape[0]
    n_s, n_h, n_r = O.regions(L)
    hist = list(range(64, 64 + n_h))
    keys, vals = [], []
    for t in range(L):
        if t in hist:
            codes, s, z = O.demote(k_bits[t:t + 1], rk, ck, group, codebook)
            keys.append(_brute_dequant(codes, s, z, group, codebook) @ rk.astype(np.float64).T)
            codes, s, z = O.demote(v_bits[t:t + 1], rv, cv, group, codebook)
            vals.append(_brute_dequant(codes, s, z, group, codebook) @ rv.astype(np.float64).T)
        elif t < n_s or t >= L - n_r:
            keys.append(O.bf16_value(k_bits[t]))
            vals.append(O.bf16_value(v_bits[t]))
    q = O.bf16_value(q_bits)
    out = np.zeros((q.shape[0], 128))
    lse = np.zeros(q.shape[0])
    for h in range(q.shape[0]):
        sc = [float(np.dot(q[h], kk)) / math.sqrt(128) for kk in keys]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        tot = math.fsum(w)
        out[h] = sum(wi * vv for wi, vv in zip(w, vals)) / tot
        lse[h] = m + math.log(tot)
    return out, lse


@pytest.mark.parametrize("L,codebook", [(L, "uniform") for L in (1, 40, 64, 65, 200, 320, 321, 333, 400)]
                         + [(L, "lloyd-max") for L in (321, 400)])
def test_request_attention_brute_force(L, codebook):
    r = rng(100 + L)
    hq, hkv, group = 4, 2, 64
    k = gen.bf16_bits(r.standard_normal((L, hkv, 128)).astype(np.float32))
    v = gen.bf16_bits(r.standard_normal((L, hkv, 128)).astype(np.float32))
    q = gen.bf16_bits(r.standard_normal((hq, 128)).astype(np.float32))
    rots = []
    for _ in range(2 * hkv):
        _, u = O.eig_descending(np.cov(r.standard_normal((300, 128)).T))
        rots.append(O.composite_rotation(u).astype(np.float32))
    rk = np.stack(rots[:hkv])
    rv = np.stack(rots[hkv:])
    ck = np.full((hkv, 128), 2.5, dtype=np.float32)
    cv = np.full((hkv, 128), 2.0, dtype=np.float32)
    out, lse = O.request_attention(q, k, v, rk, rv, ck, cv, group, codebook)
    g = hq // hkv
    for j in range(hkv):
        bo, bl = _brute_request(q[j * g:(j + 1) * g], k[:, j], v[:, j], rk[j], rv[j], ck[j], cv[j], group,
                                codebook)
        assert np.abs(out[j * g:(j + 1) * g] - bo).max() < 1e-11
        assert np.abs(lse[j * g:(j + 1) * g] - bl).max() < 1e-11


@pytest.mark.parametrize("L", [1, 7, 16])
def test_bf16_cache_attention_brute_force(L):
    """The all-bf16 baseline attention against explicit loops (fsum, math.exp)."""
    r = rng(300 + L)
    q = gen.bf16_bits(r.standard_normal((3, 128)).astype(np.float32))
    k = gen.bf16_bits((r.standard_normal((L, 128)) * 2).astype(np.float32))
    v = gen.bf16_bits(r.standard_normal((L, 128)).astype(np.float32))
    out, lse = O.bf16_cache_attention(q, k, v)
    qv, kv, vv = O.bf16_value(q), O.bf16_value(k), O.bf16_value(v)
    for h in range(3):
        sc = [math.fsum(qv[h, c] * kv[t, c] for c in range(128)) / math.sqrt(128) for t in range(L)]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        tot = math.fsum(w)
        ref = np.array([math.fsum(w[t] * vv[t, c] for t in range(L)) / tot for c in range(128)])
        assert np.abs(out[h] - ref).max() < 1e-12
        assert abs(lse[h] - (m + math.log(tot))) < 1e-12


def test_bf16_cache_attention_is_request_attention_without_history():
    """Up to 320 tokens the INT2 cache holds everything in bf16, so the two
    oracle routes must agree exactly there."""
    r = rng(301)
    L, hkv, g = 300, 2, 3
    k = gen.bf16_bits(r.standard_normal((L, hkv, 128)).astype(np.float32))
    v = gen.bf16_bits(r.standard_normal((L, hkv, 128)).astype(np.float32))
    q = gen.bf16_bits(r.standard_normal((hkv * g, 128)).astype(np.float32))
    eye = np.broadcast_to(np.eye(128, dtype=np.float32), (hkv, 128, 128)).copy()
    clip = np.full((hkv, 128), 10.0, dtype=np.float32)
    out, lse = O.request_attention(q, k, v, eye, eye, clip, clip, 128)
    for j in range(hkv):
        o2, l2 = O.bf16_cache_attention(q[j * g:(j + 1) * g], k[:, j], v[:, j])
        assert np.abs(out[j * g:(j + 1) * g] - o2).max() < 1e-13
        assert np.abs(lse[j * g:(j + 1) * g] - l2).max() < 1e-13


def test_split_merge_equals_single_softmax():
    r = rng(16)
    q = r.standard_normal((3, 128))
    k = r.standard_normal((500, 128)) * 2
    v = r.standard_normal((500, 128))
    full, full_lse = O.partial_attend(q, k, v)
    cuts = [0, 1, 64, 64, 200, 499, 500]   # includes an empty piece
    parts = [O.partial_attend(q, k[a:b], v[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    merged, merged_lse = O.merge_lse([p[0] for p in parts], [p[1] for p in parts])
    assert np.abs(merged - full).max() < 1e-13
    assert np.abs(merged_lse - full_lse).max() < 1e-12


def test_regions():
    assert O.regions(1024) == (64, 704, 256)
    assert O.regions(10) == (10, 0, 0)
    assert O.regions(64) == (64, 0, 0)
    assert O.regions(100) == (64, 0, 36)
    assert O.regions(320) == (64, 0, 256)
    assert O.regions(321) == (64, 1, 256)
    for L in range(1, 2000, 37):
        assert sum(O.regions(L)) == L


# -------------------------------------------------------------------- P11
def test_page_figures():
    fig = json.load(open(GOLDEN))
    assert O.SINK == fig["sink_tokens"]["value"]
    assert O.RECENT == fig["recent_tokens"]["value"]
    assert O.LEVELS == fig["levels"]["value"]
    assert O.CODES_PER_BYTE == fig["codes_per_byte"]["value"]
    f = fig["bf16_share_pct_at_128k"]
    assert round(100 * O.BF16_TOKENS / f["L"], f["decimals"]) == f["value"]
    for key in ("bits_per_element_128k", "bits_per_element_32k"):
        f = fig[key]
        assert round(O.bits_per_element(f["L"], f["group"]), f["decimals"]) == f["value"]
    f = fig["history_memory_reduction"]
    assert O.history_memory_ratio(128, with_metadata=False) == f["value"]
    assert 7.0 < O.history_memory_ratio(128) < f["value"]


def test_plausible_mistakes_fail_a_pin():
    """Planted mistakes in copies of oracle steps are caught by the pins' checks."""
    y = rng(17).standard_normal((200, 128)).astype(np.float32)
    codes, s, z = O.quantize_groups(y, 128)
    # scale over four levels instead of three -> max no longer on level 3
    bad_s = O.bf16_round((y.max(axis=1) - y.min(axis=1)) / np.float32(4))[:, None]
    bad = np.clip(np.rint((y - z) / bad_s), 0, 3)
    assert not np.array_equal(bad, codes)
    # H^T U P in place of U H P breaks the uniform diagonal closed form
    x = rng(18).standard_normal((300, 128)) * np.exp(rng(19).standard_normal(128))
    c = x.T @ x / 300
    _, u = O.eig_descending(c)
    wrong = O.hadamard() @ u.T @ O.bit_reversal_matrix()
    assert np.abs(np.diag(wrong.T @ c @ wrong) - np.trace(c) / 128).max() > 1e-3 * np.trace(c)


# ------------------------------------------------------------ Lloyd-Max codebook
# Pins of the codebook variant against the textbook solution and its
# optimality conditions (J. Max, "Quantizing for minimum distortion", IRE
# Transactions on Information Theory IT-6, 1960, Table I for the normal
# distribution, N = 4: output levels 0.4528 and 1.510, decision level
# 0.9816, mean squared error 0.1175).

def test_lloyd_max_matches_the_published_four_level_normal_quantizer():
    lev, thr = O.lloyd_max_gaussian(4)
    assert np.array_equal(lev, -lev[::-1]) and thr[1] == 0.0
    assert abs(lev[2] - 0.4528) < 5e-5 and abs(lev[3] - 1.510) < 5e-4
    assert abs(thr[2] - 0.9816) < 5e-5


def _normal_cell_moments(a, b):
    from scipy import integrate
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    m0 = integrate.quad(pdf, a, b, epsabs=1e-14, epsrel=1e-13)[0]
    m1 = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
    return m0, m1


def _normal_mse(levels, thresholds):
    from scipy import integrate
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    edges = [-math.inf] + list(thresholds) + [math.inf]
    return sum(integrate.quad(lambda x, y=y: (x - y) ** 2 * pdf(x), a, b, epsabs=1e-14, epsrel=1e-12)[0]
               for a, b, y in zip(edges[:-1], edges[1:], levels))


@pytest.mark.parametrize("n", [2, 4, 8])
def test_lloyd_max_satisfies_centroid_and_nearest_neighbour_conditions(n):
    """Each level is the mean of N(0,1) on its cell (quadrature, not the
    closed form the oracle uses) and each threshold is equidistant from its
    two levels; the two-level case is the closed form +-sqrt(2/pi)."""
    lev, thr = O.lloyd_max_gaussian(n)
    edges = [-math.inf] + list(thr) + [math.inf]
    for a, b, y in zip(edges[:-1], edges[1:], lev):
        m0, m1 = _normal_cell_moments(a, b)
        assert abs(m1 / m0 - y) < 1e-9
    assert np.allclose(thr, (lev[:-1] + lev[1:]) / 2, rtol=0, atol=1e-15)
    if n == 2:
        assert abs(lev[1] - math.sqrt(2 / math.pi)) < 1e-14


def test_lloyd_max_is_a_local_minimum_of_the_distortion():
    lev, thr = O.lloyd_max_gaussian(4)
    d0 = _normal_mse(lev, thr)
    assert abs(d0 - 0.1175) < 5e-5
    # the best uniform 4-level quantizer of N(0,1) (step ~0.996) is worse
    from scipy import optimize
    uni = optimize.minimize_scalar(lambda d: _normal_mse(np.array([-1.5, -0.5, 0.5, 1.5]) * d,
                                                         np.array([-1.0, 0.0, 1.0]) * d),
                                   bounds=(0.5, 1.5), method="bounded")
    assert uni.fun > d0 + 1e-3
    for dl in (-1e-3, 1e-3):
        for i in range(4):
            l2 = lev.copy()
            l2[i] += dl
            assert _normal_mse(l2, thr) > d0
        for i in (0, 2):
            t2 = thr.copy()
            t2[i] += dl
            assert _normal_mse(lev, t2) > d0


@pytest.mark.parametrize("group", [32, 64, 128])
def test_lloyd_quantizer_statistics_brute_force_and_bound(group):
    r = rng(40 + group)
    n = 300
    y = (r.standard_normal((n, 128)) * np.exp(r.standard_normal(128)) + r.standard_normal(128)).astype(np.float32)
    codes, s, z = O.quantize_groups_lloyd(y, group)
    ng = 128 // group
    assert codes.dtype == np.uint8 and codes.max() <= 3
    assert np.array_equal(O.bf16_round(s), s) and np.array_equal(O.bf16_round(z), z)
    yg = y.reshape(n, ng, group)
    import statistics
    lev32, thr32 = O.lloyd_max_codebook()
    for t in range(0, n, 7):
        for gi in range(ng):
            vals = [float(x) for x in yg[t, gi]]
            # statistics computes the mean and population deviation exactly (rationals)
            assert z[t, gi] == O.bf16_round(np.float32(statistics.fmean(vals)))
            assert s[t, gi] == O.bf16_round(np.float32(statistics.pstdev(vals)))
            for c in range(group):
                u = float(np.float32(np.float32(yg[t, gi, c] - z[t, gi]) / s[t, gi]))
                dist = [abs(u - float(l)) for l in lev32]
                best = int(np.argmin(dist))
                if min(abs(u - float(th)) for th in thr32) > 1e-6:
                    assert codes[t, gi * group + c] == best
    yhat = O.dequantize_lloyd(codes, s, z, group).reshape(n, ng, group)
    # error bound: the largest half cell inside the outer levels, or the
    # distance past the outer level
    u = (yg - z[..., None]) / s[..., None]
    inner = np.abs(u) <= lev32[3]
    half_gap = max((lev32[1] - lev32[0]) / 2, (lev32[2] - lev32[1]) / 2)
    err = np.abs(yhat - yg) / s[..., None]
    assert (err[inner] <= half_gap + 1e-5).all()
    assert np.allclose(err[~inner], np.abs(u[~inner]) - lev32[3], atol=1e-5)


def test_lloyd_quantizer_mirror_constant_group_and_gaussian_distortion():
    r = rng(44)
    y = (r.standard_normal((200, 128)) * 3 + 1).astype(np.float32)
    c1, s1, z1 = O.quantize_groups_lloyd(y, 64)
    c2, s2, z2 = O.quantize_groups_lloyd(-y, 64)
    assert np.array_equal(s1, s2) and np.array_equal(z1, -z2)
    assert np.array_equal(c2, 3 - c1)
    # constant group: scale 0, code 0, exact reconstruction of the bf16 value
    yc = np.full((2, 128), 0.3, dtype=np.float32)
    c, s, z = O.quantize_groups_lloyd(yc, 32)
    assert (c == 0).all() and (s == 0).all()
    assert np.array_equal(O.dequantize_lloyd(c, s, z, 32), np.broadcast_to(O.bf16_round(yc), yc.shape))
    # Gaussian groups: relative distortion near the codebook's 0.1175, well
    # under the min/max uniform quantizer's on the same data
    g = r.standard_normal((4000, 128)).astype(np.float32)
    c, s, z = O.quantize_groups_lloyd(g, 128)
    yh = O.dequantize_lloyd(c, s, z, 128)
    var = g.astype(np.float64).var(axis=1)
    d_lm = (((yh - g) ** 2).mean(axis=1) / var).mean()
    cu, su, zu = O.quantize_groups(g, 128)
    yu = O.dequantize(cu, su, zu, 128).astype(np.float64)
    d_u = (((yu - g) ** 2).mean(axis=1) / var).mean()
    assert abs(d_lm - 0.1175) < 0.006
    assert d_u > 1.5 * d_lm
