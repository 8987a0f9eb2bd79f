"""GPU parity of the all-bf16 KV-cache baseline (split-K decode over bf16
pages, merge, append) against the oracle's float64 attention over the same
bf16 tokens.  Bar: 2e-3 max-abs and 1e-3 relative L2 on the output, 2e-3 on
the LSE (the same bar as the INT2 path)."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_split_amd as ok
from bit_rotated_kv_split_amd import workload as W
from oracle import oscar as O
from synth import configs, gen

from gpu_helpers import assert_close, request_tokens

pytestmark = pytest.mark.gpu


def small(name, seed, hq, hkv, lens, paged=True):
    return configs.Workload(name, seed, hq, hkv, 128, len(lens), tuple(lens), paged=paged,
                            shared_prefix=False, anisotropic_q=True)


def run(cache, q, max_len, target=0):
    opts = ok.make_options(history_target=target) if target else None
    nb = ok.oscar_bf16_decode_workspace_bytes(cache.dims, cache.batch)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.full((cache.batch, cache.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((cache.batch, cache.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    ok.oscar_bf16_decode(cache.dims, cache.struct(), q, max_len, ws, nb, out, lse, options=opts)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(w, layout, model, out, lse, requests=None):
    g = w.num_q_heads // w.num_kv_heads
    qb = model.queries(0, w.batch)
    for b in (range(w.batch) if requests is None else requests):
        L = int(layout.lens[b])
        k, v = request_tokens(model, layout, b, L)
        for j in range(w.num_kv_heads):
            ref, ref_lse = O.bf16_cache_attention(qb[b, j * g:(j + 1) * g], k[:, j], v[:, j])
            assert_close(out[b, j * g:(j + 1) * g], ref, f"{w.name} b={b} L={L} kvh={j}")
            assert np.abs(lse[b, j * g:(j + 1) * g] - ref_lse).max() < 2e-3


@pytest.mark.parametrize("gqa", [1, 4, 8])
@pytest.mark.parametrize("target", [0, 1])
def test_baseline_matches_oracle(gqa, target):
    lens = [1, 63, 64, 65, 320, 1000, 5000]
    w = small(f"base{gqa}", 120 + gqa, 2 * gqa, 2, lens)
    layout = W.Layout(w)
    model = W.SyntheticModel(w)
    cache = W.build_bf16_cache(w, layout)
    q = W.queries_tensor(model, 0, w.batch)
    out, lse = run(cache, q, max(lens), target)
    check(w, layout, model, out, lse)


def test_baseline_append_then_decode():
    lens = [63, 64, 2000]
    w = small("baseapp", 130, 8, 2, lens)
    layout = W.Layout(w)
    model = W.SyntheticModel(w)
    cache = W.build_bf16_cache(w, layout, extra_tokens=1)
    lens1 = layout.lens + 1
    cache.seq_lens.copy_(torch.from_numpy(lens1.astype(np.int32)))
    kn = W.new_tokens_tensor(model, layout, lens1, "k")
    vn = W.new_tokens_tensor(model, layout, lens1, "v")
    ok.oscar_bf16_append(cache.dims, cache.struct(), kn, vn)
    layout.lens = lens1
    q = W.queries_tensor(model, 0, w.batch)
    out, lse = run(cache, q, int(lens1.max()))
    check(w, layout, model, out, lse)


@pytest.mark.slow
def test_baseline_full_size_sampled():
    """32 x 100K, 32 q / 8 kv heads, in the launch configuration bench.py
    times (12.8 GB of bf16 pages); three (request, KV head) groups checked."""
    w = configs.qwen3_8b_b32(128)
    layout = W.Layout(w)
    model = W.SyntheticModel(w)
    cache = W.build_bf16_cache(w, layout)
    q = W.queries_tensor(model, 0, w.batch)
    out, lse = run(cache, q, int(layout.lens.max()))
    g = w.num_q_heads // w.num_kv_heads
    qb = model.queries(0, w.batch)
    for b, j in [(0, 0), (17, 5), (31, 7)]:
        L = int(layout.lens[b])
        k = np.stack([gen.kv_tokens_bf16(w.seed, "k", b, j, 0, L, model.k_scale[j])], 1)
        v = np.stack([gen.kv_tokens_bf16(w.seed, "v", b, j, 0, L, model.v_scale[j])], 1)
        ref, ref_lse = O.bf16_cache_attention(qb[b, j * g:(j + 1) * g], k[:, 0], v[:, 0])
        assert_close(out[b, j * g:(j + 1) * g], ref, f"full b={b} kvh={j}")
        assert np.abs(lse[b, j * g:(j + 1) * g] - ref_lse).max() < 2e-3
