"""Rotation ablation on seeded synthetic data: INT2 decode attention with
different rotations against the all-bf16 cache, on the GPU.

    python -m bit_rotated_kv_split_amd.ablation [--batch 4] [--context 32768] [--seed 11] [--groups 128,64,32]
        [--q-scales 0.0625,0.25,1]

The pages compare OSCAR's attention-aware rotation with no rotation (naive
INT2) and with fixed Hadamard rotations (page "Together AI 开源 OSCAR…",
sections "为什么 INT2 KV 缓存量化很难？" and "结果"; page "超越TurboQuant…",
section "OSCAR把旋转对准attention").  Their quality numbers come from model
accuracy suites that are not reproduced here; this measures the same
ordering on a synthetic stand-in: the relative L2 error of each query
head's attention output, and the absolute error of its log-sum-exp, against
the same decode over an all-bf16 cache of the same tokens.

Rotation sets (every one clipped per channel at the calibration data's
99.9th percentile of |x R|, as OSCAR is; "oscar-noclip" drops the clip):
  identity        R = I
  hadamard        R = H (normalised Sylvester)
  hadamard-bitrev R = H P (H then the 7-bit bit-reversal permutation)
  oscar           R_K = U_Q H P, R_V = U_S H P from oscar_calibrate
  oscar-noclip    the same rotations, no clipping
  oscar-lloyd-max OSCAR's rotations with the Lloyd-Max codebook (levels of
                  N(0, 1) on mean/deviation-normalised groups) in place of
                  the uniform min/max levels

The generator's raw queries (q-scale 1) give attention logits with a
standard deviation near 10 over a 32K context, so each head attends to a
handful of tokens and any INT2 error that reorders them dominates; the
query scale (a power of two, exact in bf16, applied to the decode queries
and to the calibration queries alike) sweeps the logit spread down to
where attention is spread over many tokens.

Quantization groups run along the channels of one token, so the bit
reversal changes nothing at G = 128 (one group per token) and interleaves
channels across groups at G = 64 and 32.  Prints one JSON line per
(group size, rotation set).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import sys

import numpy as np


def sylvester_hadamard(n: int = 128) -> np.ndarray:
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(n)


def bit_reversal_perm(n: int = 128) -> np.ndarray:
    bits = n.bit_length() - 1
    idx = np.array([int(f"{i:0{bits}b}"[::-1], 2) for i in range(n)])
    p = np.zeros((n, n))
    p[np.arange(n), idx] = 1.0          # (x P)_k = x_{bitrev(k)}: P[bitrev(k)][k] = 1, P symmetric
    return p


def clips_for(x: np.ndarray, r: np.ndarray, pct: float) -> np.ndarray:
    """Per-channel pct-th percentile of |x R| over the calibration tokens, per KV head."""
    hkv = r.shape[0]
    return np.stack([np.percentile(np.abs(x[:, j].astype(np.float64) @ r[j].astype(np.float64)), pct, axis=0)
                     for j in range(hkv)]).astype(np.float32)


def logit_error(ok, W, cache, w, layout, model, r_k, q_bits, q_scale: float, n_tok: int) -> float:
    """Mean over (request, KV head) of ||Q (K_hat - K)^T||^2 / ||Q K^T||^2 on
    history indices 0 .. n_tok-1 (float64 on the host)."""
    import torch
    from synth import gen
    B, hkv, g = w.batch, w.num_kv_heads, w.gqa
    ko = torch.empty((n_tok, hkv, 128), dtype=torch.float32, device="cuda")
    vo = torch.empty_like(ko)
    r = r_k.cpu().numpy() if hasattr(r_k, "cpu") else np.asarray(r_k)
    ratios = []
    for b in range(B):
        ok.oscar_kv_read_history(cache.dims, cache.struct(), b, 0, n_tok, ko, vo)
        torch.cuda.synchronize()
        kh = ko.cpu().numpy().astype(np.float64)
        for j in range(hkv):
            k = np.zeros((n_tok, 128), dtype=np.uint16)
            for src, p0, n in layout.src_ranges(b, ok.SINK, n_tok):
                k[p0 - ok.SINK:p0 - ok.SINK + n] = gen.kv_tokens_bf16(w.seed, "k", src, j, p0, n, model.k_scale[j])
            kf = (k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            k_hat = kh[:, j] @ r[j].astype(np.float64).T
            q = (q_bits[b, j * g:(j + 1) * g].astype(np.uint32) << 16).view(np.float32).astype(np.float64) * q_scale
            ref = q @ kf.T
            ratios.append(float(np.sum((q @ k_hat.T - ref) ** 2) / np.sum(ref ** 2)))
    return float(np.mean(ratios))


def run(batch: int = 4, context: int = 32768, seed: int = 11, q_heads: int = 32, kv_heads: int = 8,
        groups=(128, 64, 32), q_scales=(0.0625, 0.25, 1.0), logit_tokens: int = 4096):
    """Yield one dict of error metrics per (query scale, group size, rotation set)."""
    import torch
    from synth import configs
    from . import _lib as ok
    from . import workload as W
    from .kvcache import DecodeWorkspace, Rotation

    groups, q_scales = list(groups), [float(x) for x in q_scales]
    for x in q_scales:
        if np.frexp(x)[0] != 0.5:
            raise ValueError(f"q-scale {x} is not a power of two")
    base = configs.Workload("ablation", seed, q_heads, kv_heads, groups[0], batch, (context,) * batch,
                            paged=True)
    model = W.SyntheticModel(base)
    layout = W.Layout(base)
    B, hq, hkv = base.batch, base.num_q_heads, base.num_kv_heads
    qc, kc, vc = model.calibration()
    q_bits = model.queries(0, B)
    q1 = W.queries_tensor(model, 0, B)
    L = int(layout.lens.max())

    # the all-bf16 reference (independent of the group size), per query scale
    dims = ok.make_dims(hq, hkv, groups[0])
    bc = W.build_bf16_cache(base, layout)
    nb = ok.oscar_bf16_decode_workspace_bytes(dims, B)
    wsb = torch.empty(nb, dtype=torch.uint8, device="cuda")
    refs = {}
    for qs in q_scales:
        ref = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
        ref_lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
        ok.oscar_bf16_decode(bc.dims, bc.struct(), (q1 * qs).contiguous(), L, wsb, nb, ref, ref_lse)
        torch.cuda.synchronize()
        refs[qs] = (ref.cpu().numpy().astype(np.float64), ref_lse.cpu().numpy().astype(np.float64))
    del bc, wsb

    h = sylvester_hadamard()
    hp = h @ bit_reversal_perm()
    fixed = {"identity": np.eye(128), "hadamard": h, "hadamard-bitrev": hp}
    fixed_sets = []
    for name, r in fixed.items():
        r3 = np.broadcast_to(r.astype(np.float32), (hkv, 128, 128)).copy()
        fixed_sets.append((name, r3, r3, clips_for(kc, r3, base.clip_pct), clips_for(vc, r3, base.clip_pct)))
    kd, vd = (torch.from_numpy(x).cuda() for x in (kc, vc))

    for qs, g in ((qs, g) for qs in q_scales for g in groups):
        qd = torch.from_numpy(qc * np.float32(qs)).cuda()
        q = (q1 * qs).contiguous()
        ref, ref_lse = refs[qs]
        w = dataclasses.replace(base, group_size=g)
        dims = ok.make_dims(hq, hkv, g)
        # OSCAR's rotations from the library
        cws = torch.empty(ok.oscar_calibrate_workspace_bytes(dims, qc.shape[0]), dtype=torch.uint8,
                          device="cuda")
        rk = torch.empty((hkv, 128, 128), dtype=torch.float32, device="cuda")
        rv = torch.empty_like(rk)
        ck = torch.empty((hkv, 128), dtype=torch.float32, device="cuda")
        cv = torch.empty_like(ck)
        ok.oscar_calibrate(dims, qc.shape[0], qd, kd, vd, w.clip_pct, rk, rv, ck, cv, None, None,
                           cws, cws.numel())
        torch.cuda.synchronize()
        del cws
        big = np.full((hkv, 128), 3.0e38, dtype=np.float32)
        sets = [s + (ok.CODEBOOK_UNIFORM,) for s in fixed_sets]
        sets += [("oscar", rk, rv, ck, cv, ok.CODEBOOK_UNIFORM), ("oscar-noclip", rk, rv, big, big, ok.CODEBOOK_UNIFORM),
                 ("oscar-lloyd-max", rk, rv, ck, cv, ok.CODEBOOK_LLOYD_MAX)]
        for name, r_k, r_v, c_k, c_v, cb in sets:
            rot = Rotation(r_k, r_v, c_k, c_v)
            wc = dataclasses.replace(w, codebook=cb)
            cache = W.build_cache(wc, layout, model, rot)
            ws = DecodeWorkspace(cache.dims, B, L)
            out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
            lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
            ok.oscar_decode(cache.dims, rot.struct, cache.struct(), q, L, ws.buf, ws.nbytes, out, lse)
            torch.cuda.synchronize()
            o = out.cpu().numpy().astype(np.float64)
            rel = np.linalg.norm(o - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
            lerr = np.abs(lse.cpu().numpy() - ref_lse)
            n_tok = min(logit_tokens, L - W.BF16_TOKENS)
            logit = logit_error(ok, W, cache, wc, layout, model, r_k, q_bits, qs, n_tok) if n_tok > 0 else 0.0
            del cache, ws
            yield {"q_scale": qs, "group_size": g, "rotation": name, "out_rel_l2_mean": float(rel.mean()),
                   "out_rel_l2_p95": float(np.percentile(rel, 95)), "out_rel_l2_max": float(rel.max()),
                   "lse_abs_err_mean": float(lerr.mean()), "lse_abs_err_max": float(lerr.max()),
                   "ref_lse_minus_log_len_mean": float((ref_lse - np.log(L)).mean()),
                   "logit_rel_err": logit, "logit_tokens": n_tok,
                   "batch": B, "context": L, "q_heads": hq, "kv_heads": hkv, "seed": seed}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--context", type=int, default=32768)
    ap.add_argument("--seed", type=int, default=11)
    ap.add_argument("--q-heads", type=int, default=32)
    ap.add_argument("--kv-heads", type=int, default=8)
    ap.add_argument("--groups", default="128,64,32")
    ap.add_argument("--q-scales", default="0.0625,0.25,1")
    ap.add_argument("--logit-tokens", type=int, default=4096)
    args = ap.parse_args(argv)
    for rec in run(args.batch, args.context, args.seed, args.q_heads, args.kv_heads,
                   [int(g) for g in args.groups.split(",")], [float(x) for x in args.q_scales.split(",")],
                   args.logit_tokens):
        print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
