"""Rotation ablation (bit_rotated_kv_split_amd/ablation.py): its fixed
rotations on the CPU and one small run on the GPU."""
import numpy as np
import pytest

from bit_rotated_kv_split_amd import ablation


def test_fixed_rotations_are_orthogonal_and_bitrev_is_an_involution():
    h = ablation.sylvester_hadamard()
    p = ablation.bit_reversal_perm()
    assert np.allclose(h @ h.T, np.eye(128), atol=1e-14)
    assert np.array_equal(p @ p, np.eye(128))
    x = np.arange(128.0)
    y = x @ p
    # (x P)_k = x_{bitrev7(k)}: channel 1 = 0b0000001 lands at 0b1000000 = 64
    assert y[64] == 1 and y[1] == 64 and y[3] == 96 and y[127] == 127


def test_clips_are_percentiles_of_rotated_magnitudes():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1000, 2, 128)).astype(np.float32)
    r = np.stack([np.eye(128), ablation.sylvester_hadamard()]).astype(np.float32)
    c = ablation.clips_for(x, r, 50.0)
    assert np.allclose(c[0], np.median(np.abs(x[:, 0]), axis=0), rtol=1e-6)
    assert np.allclose(c[1], np.median(np.abs(x[:, 1].astype(np.float64) @ r[1]), axis=0), rtol=1e-6)


@pytest.mark.gpu
def test_rotation_ablation_orders_naive_int2_last():
    recs = {r["rotation"]: r for r in ablation.run(batch=2, context=8192, groups=(64,), q_scales=(0.0625,),
                                                   logit_tokens=1024)}
    assert set(recs) == {"identity", "hadamard", "hadamard-bitrev", "oscar", "oscar-noclip", "oscar-lloyd-max"}
    for name in ("hadamard", "hadamard-bitrev", "oscar", "oscar-lloyd-max"):
        assert recs[name]["out_rel_l2_mean"] < 0.75 * recs["identity"]["out_rel_l2_mean"], name
        assert recs[name]["lse_abs_err_mean"] < recs["identity"]["lse_abs_err_mean"], name
    assert all(np.isfinite(r["out_rel_l2_max"]) for r in recs.values())
    # the pages' key objective: rotation lowers the relative logit error too
    for name in ("hadamard", "oscar", "oscar-lloyd-max"):
        assert recs[name]["logit_rel_err"] < 0.5 * recs["identity"]["logit_rel_err"], name
    assert all(0 < r["logit_rel_err"] < 10 for r in recs.values())
