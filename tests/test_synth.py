"""The seeded input generator: determinism, exactness and distribution."""
import numpy as np

from synth import gen


def test_deterministic_and_counter_based():
    k = gen.stream_key(5, gen.STREAM_K_CACHE)
    a = gen.rand64(k, np.arange(1000, dtype=np.uint64))
    b = gen.rand64(k, np.arange(500, 1000, dtype=np.uint64))
    assert np.array_equal(a[500:], b)
    assert gen.stream_key(5, 1) != gen.stream_key(5, 2) != gen.stream_key(6, 1)


def test_splitmix_finaliser_is_a_bijection_on_samples():
    x = np.arange(1 << 16, dtype=np.uint64) * np.uint64(0x10001)
    assert np.unique(gen.mix64(x)).size == x.size


def test_normal_is_exact_dyadic_and_standard():
    k = gen.stream_key(1, gen.STREAM_V_CACHE)
    x = gen.normal_f32(k, np.arange(1_000_000, dtype=np.uint64))
    assert x.dtype == np.float32
    scaled = x.astype(np.float64) * 65536
    assert np.array_equal(scaled, np.round(scaled))
    assert abs(x.mean()) < 3e-3 and abs(x.std() - 1) < 3e-3
    assert 2.8 < ((x / x.std()) ** 4).mean() < 3.0
    assert np.abs(x).max() <= 6.0


def test_kv_tokens_outliers_and_bf16():
    ks, vs = gen.outlier_scales(0, 2)
    assert (ks == 20).sum(axis=1).tolist() == [4, 4]
    assert (vs == 10).sum(axis=1).tolist() == [2, 2]
    f = gen.kv_tokens_f32(0, "k", 3, 1, 100, 50, ks[1])
    b = gen.kv_tokens_bf16(0, "k", 3, 1, 100, 50, ks[1])
    assert np.array_equal(gen.bf16_to_f32(b), gen.bf16_to_f32(gen.bf16_bits(f)))
    # any sub-range of positions reproduces the same tokens
    assert np.array_equal(gen.kv_tokens_bf16(0, "k", 3, 1, 120, 10, ks[1]), b[20:30])


def test_permutation_and_lengths():
    p = gen.permutation(2, 1000)
    assert sorted(p.tolist()) == list(range(1000))
    L = gen.ragged_lengths(4, 32, 4096, 131072)
    assert L.min() >= 4096 and L.max() <= 131072
