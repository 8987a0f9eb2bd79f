"""oscar_decode_step_noalloc (the library's own per-device scratch as the
workspace) against oscar_decode_step with a caller-allocated workspace: the
same output and LSE bits and the same cache bytes afterwards, on two calls
in a row, the second with a smaller batch, fewer heads and shorter lengths
(the scratch then holds the first call's contents)."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_split_amd as ok
from bit_rotated_kv_split_amd import workload as W
from bit_rotated_kv_split_amd.kvcache import DecodeWorkspace, Rotation
from synth import configs

from gpu_helpers import oracle_calibration

pytestmark = pytest.mark.gpu


def _case(name, seed, hq, hkv, group, lens, codebook=0):
    w = configs.Workload(name, seed, hq, hkv, group, len(lens), tuple(lens), paged=True, codebook=codebook)
    layout = W.Layout(w, None, extra_tokens=1)
    model = W.SyntheticModel(w)
    cal = oracle_calibration(model)
    rot = Rotation(cal["r_k32"], cal["r_v32"], cal["clip_k"], cal["clip_v"])
    cache = W.build_cache(w, layout, model, rot)
    lens1 = layout.lens + 1
    cache.seq_lens.copy_(torch.from_numpy(lens1.astype(np.int32)))
    kn = W.new_tokens_tensor(model, layout, lens1, "k")
    vn = W.new_tokens_tensor(model, layout, lens1, "v")
    q = W.queries_tensor(model, 1, w.batch)
    return w, cache, rot, kn, vn, q, int(lens1.max())


def _state(cache):
    return [t.clone() for t in (cache.pages, cache.sink_k, cache.sink_v, cache.recent_k, cache.recent_v)]


def _restore(cache, snap):
    for t, s0 in zip((cache.pages, cache.sink_k, cache.sink_v, cache.recent_k, cache.recent_v), snap):
        t.copy_(s0)


def _check(case):
    w, cache, rot, kn, vn, q, max_len = case
    print(f"[noalloc] {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} G={w.group_size} "
          f"max_len={max_len}", flush=True)
    before = _state(cache)
    out_a = torch.full((w.batch, w.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse_a = torch.full((w.batch, w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    ok.oscar_decode_step_noalloc(cache.dims, rot.struct, cache.struct(), kn, vn, q, max_len, out_a, lse_a)
    torch.cuda.synchronize()
    after_a = _state(cache)
    _restore(cache, before)
    ws = DecodeWorkspace(cache.dims, w.batch, max_len)
    out_b = torch.full_like(out_a, float("nan"))
    lse_b = torch.full_like(lse_a, float("nan"))
    ok.oscar_decode_step(cache.dims, rot.struct, cache.struct(), kn, vn, q, max_len, ws.buf, ws.nbytes, out_b,
                         lse_b)
    torch.cuda.synchronize()
    assert torch.isfinite(out_a).all()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    for ta, tb in zip(after_a, _state(cache)):
        assert torch.equal(ta, tb)


def test_noalloc_step_equals_step_with_workspace_on_two_calls():
    _check(_case("noalloc-a", 90, 16, 2, 128, [9000, 4000, 321, 700, 12000, 64]))
    _check(_case("noalloc-b", 91, 4, 1, 64, [2000, 500], codebook=ok.CODEBOOK_LLOYD_MAX))
