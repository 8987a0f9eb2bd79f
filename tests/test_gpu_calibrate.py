"""GPU parity of the offline calibration (C_Q, C_S, R = U.H.P_br, clip
percentiles) against the oracle.

Eigenvectors are unique (up to the fixed sign convention) only where the
eigenvalue gap is large; columns are compared one by one under a
perturbation bound set by the gap, and the decomposition itself is checked
for every column."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_split_amd as ok
from bit_rotated_kv_split_amd.workload import SyntheticModel
from oracle import oscar as O
from synth import configs

pytestmark = pytest.mark.gpu


def run_gpu_calibration(model):
    w = model.w
    q, k, v = model.calibration()
    dims = ok.make_dims(w.num_q_heads, w.num_kv_heads, w.group_size)
    n = q.shape[0]
    ws_bytes = ok.oscar_calibrate_workspace_bytes(dims, n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    hkv = w.num_kv_heads
    r_k = torch.empty((hkv, 128, 128), dtype=torch.float32, device="cuda")
    r_v = torch.empty_like(r_k)
    c_k = torch.empty((hkv, 128), dtype=torch.float32, device="cuda")
    c_v = torch.empty_like(c_k)
    rk64 = np.zeros((hkv, 128, 128))
    rv64 = np.zeros((hkv, 128, 128))
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    ok.oscar_calibrate(dims, n, qd, kd, vd, w.clip_pct, r_k, r_v, c_k, c_v, rk64, rv64, ws, ws_bytes)
    return (q, k, v), rk64, rv64, r_k.cpu().numpy(), r_v.cpu().numpy(), c_k.cpu().numpy(), c_v.cpu().numpy()


def eigvecs_of_rotation(r):
    """U = R P H (inverse of R = U H P for symmetric orthogonal H and P)."""
    return r @ O.bit_reversal_matrix() @ O.hadamard()


def check_rotation(r_gpu, r_ref, c, lam_ref, what):
    assert np.abs(r_gpu.T @ r_gpu - np.eye(128)).max() <= 1e-10, what
    u_gpu = eigvecs_of_rotation(r_gpu)
    u_ref = eigvecs_of_rotation(r_ref)
    scale = lam_ref[0]
    # every column is an eigenvector with the oracle's eigenvalue, in order
    resid = c @ u_gpu - u_gpu * lam_ref[None, :]
    assert np.abs(resid).max() <= 1e-9 * scale, what
    gaps = np.full(128, np.inf)
    gaps[:-1] = np.minimum(gaps[:-1], lam_ref[:-1] - lam_ref[1:])
    gaps[1:] = np.minimum(gaps[1:], lam_ref[:-1] - lam_ref[1:])
    compared = 0
    for j in range(128):
        bound = 1e-10 + 1e-13 * scale / max(gaps[j], 1e-300)
        if bound < 1e-3:
            assert np.abs(u_gpu[:, j] - u_ref[:, j]).max() <= bound, f"{what} col {j}"
            compared += 1
    return compared


@pytest.mark.parametrize("which", ["tiny", "gqa4-anisotropic"])
def test_calibration_matches_oracle(which):
    if which == "tiny":
        w = configs.tiny()
    else:
        w = configs.Workload("cal4", 12, 8, 2, 128, 1, (1000,))
    model = SyntheticModel(w)
    (q, k, v), rk64, rv64, rk32, rv32, ck, cv = run_gpu_calibration(model)
    cal = O.calibrate(q, k, v, w.clip_pct)
    g = w.gqa
    n_cmp = 0
    for j in range(w.num_kv_heads):
        cq = O.query_covariance(q[:, j * g:(j + 1) * g])
        cs = O.score_weighted_value_covariance(q[:, j * g:(j + 1) * g], k[:, j], v[:, j])
        n_cmp += check_rotation(rk64[j], cal["r_k"][j], cq, cal["lam_q"][j], f"R_K kvh={j}")
        n_cmp += check_rotation(rv64[j], cal["r_v"][j], cs, cal["lam_s"][j], f"R_V kvh={j}")
        # uniform-diagonal closed form holds for the library's rotations too
        for r, c in ((rk64[j], cq), (rv64[j], cs)):
            d = np.diag(r.T @ c @ r)
            assert np.abs(d - np.trace(c) / 128).max() <= 1e-10 * np.trace(c)
    assert n_cmp >= 64 * w.num_kv_heads
    assert np.array_equal(rk32, rk64.astype(np.float32))
    assert np.array_equal(rv32, rv64.astype(np.float32))
    # clip thresholds: percentiles of |x R| recomputed with the library's own
    # rotation, to the last float32 bit (up to one ulp of interpolation order)
    for j in range(w.num_kv_heads):
        for x, r, got in ((k[:, j], rk64[j], ck[j]), (v[:, j], rv64[j], cv[j])):
            ref = O.clip_thresholds(x, r, w.clip_pct)
            assert np.all(np.abs(got - ref) <= np.spacing(ref)), np.abs(got - ref).max()
        assert np.allclose(ck[j], cal["clip_k"][j], rtol=1e-6, atol=0)
        assert np.allclose(cv[j], cal["clip_v"][j], rtol=1e-6, atol=0)


def test_calibration_rejects_bad_arguments():
    dims = ok.make_dims(8, 2, 128)
    assert ok.oscar_calibrate_workspace_bytes(dims, 1) == 0
    assert ok.oscar_calibrate_workspace_bytes(dims, ok.oscar_calibrate_max_tokens() + 1) == 0
    with pytest.raises(ok.OscarError):
        ok.oscar_calibrate(dims, 100, 0x1000, 0x1000, 0x1000, 150.0, 0x1000, 0x1000, 0x1000, 0x1000,
                           None, None, 0x1000, 1 << 30)
