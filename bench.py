#!/usr/bin/env python3
"""Decode-step benchmark of the OSCAR INT2 KV-cache path on one MI355X.

A step is one pass of the whole hot path over the batch (oscar_decode_step):
append + demotion, query rotation and the split schedule in one launch; INT2
history split-K + bf16 sink/recent in a second; LSE merge + value
un-rotation in a third.  Inputs
(cache, queries, new tokens, lengths) are resident in HBM before timing
starts; every step appends one token per request, so lengths grow by one.

Default workload: 32 requests at 100K context, 32 query / 8 KV heads,
head_dim 128, G = 128, paged cache (64-token pages, seeded random page
permutation), synthetic seeded data; rotations and clips calibrated by the
library from a synthetic calibration sequence before timing.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "decode-attn µs/step + achieved HBM GB/s (% peak), 100K ctx, batch 32"


def workloads():
    from synth import configs, gen
    return {
        "b32-100k-g128": lambda: configs.qwen3_8b_b32(128),
        "b32-100k-g64": lambda: configs.qwen3_8b_b32(64),
        "b1-100k": lambda: configs.qwen3_8b_b1(),
        "b16-128k": lambda: configs.qwen3_4b_b16(),
        "b32-ragged-gqa8": lambda: configs.qwen3_32b_ragged(
            tuple(int(x) for x in gen.ragged_lengths(4, 32, 4096, 131072))),
    }


def hist_unit_bytes(group: int) -> int:
    """Algorithmic bytes per history token per KV head: 2 x 32 code bytes and
    2 x (128/G) bf16 (scale, zero) pairs."""
    return 2 * 32 + 2 * (128 // group) * 4


def bf16_bytes(lens: np.ndarray, hkv: int) -> int:
    """Algorithmic bytes of the bf16 sink/recent tokens: 512 per token and KV head."""
    return int(np.minimum(lens, 320).sum()) * hkv * 2 * 128 * 2


def step_bytes(lens: np.ndarray, hkv: int, hq: int, group: int) -> tuple[int, int]:
    """(history bytes, whole-step bytes) the method must move for one step at
    the given lengths: history codes + scale/zero, bf16 sink/recent tokens,
    queries in and outputs out, and the demoted/appended tokens."""
    n_hist = np.maximum(lens - 320, 0)
    n_bf16 = np.minimum(lens, 320)
    hist = int(n_hist.sum()) * hkv * hist_unit_bytes(group)
    bf16 = int(n_bf16.sum()) * hkv * 2 * 128 * 2
    qo = len(lens) * hq * 128 * (2 + 4)
    demoted = int((lens > 320).sum()) * hkv * (2 * 256 + hist_unit_bytes(group))
    appended = len(lens) * hkv * 2 * 256
    return hist, hist + bf16 + qo + demoted + appended


def load_traffic(workload: str, kernel: str):
    """HBM bytes per history-kernel launch from the committed rocprofv3 PMC
    summary, or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{workload}/{kernel}")
    except (OSError, ValueError):
        return None
    from bit_rotated_kv_split_amd.profiling import source_sha
    if not rec or rec.get("source_sha") != source_sha(ROOT):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(model, layout, cal_host, lens, n_heads: int, budget_s: float = 10.0):
    """Time the oracle (as it stands) on whole requests of the same workload
    at their final length, request 0 first, until about budget_s seconds of
    oracle work; scaled to GB/s of the same algorithmic bytes.  The sample's
    tokens come from the GPU twin of the seeded generator (bit-identical to
    synth.gen; not timed)."""
    import torch
    from oracle import oscar as O
    from synth import gpu as synth_gpu
    w = model.w
    g = w.gqa
    stream = torch.cuda.current_stream().cuda_stream
    spent = 0.0
    done_bytes = 0
    reqs = 0
    for b in range(w.batch):
        L = int(lens[b])
        host = {}
        for which, scale in (("k", model.k_scale), ("v", model.v_scale)):
            buf = torch.empty((L, n_heads, 128), dtype=torch.int16, device="cuda")
            sc = torch.from_numpy(np.ascontiguousarray(scale[:n_heads])).cuda()
            for src, p0, n in layout.src_ranges(b, 0, L):
                synth_gpu.fill_kv(buf.data_ptr() + 2 * p0 * n_heads * 128, n, n_heads, n_heads * 128, 128,
                                  w.seed, which, src, p0, sc, stream)
            torch.cuda.synchronize()
            host[which] = buf.cpu().numpy().view(np.uint16)
            del buf
        q = model.queries(0, w.batch)[b][: n_heads * g]
        t0 = time.perf_counter()
        O.request_attention(q, host["k"], host["v"], cal_host["r_k32"][:n_heads], cal_host["r_v32"][:n_heads],
                            cal_host["clip_k"][:n_heads], cal_host["clip_v"][:n_heads], w.group_size)
        spent += time.perf_counter() - t0
        done_bytes += step_bytes(np.array([L]), n_heads, n_heads * g, w.group_size)[1]
        reqs += 1
        if spent >= budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:
        cores = 1
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seconds": round(spent, 3),
            "sample": f"requests 0..{reqs - 1} of {w.batch}, {n_heads} of {w.num_kv_heads} KV heads each, "
                      f"at their final lengths: the oracle demotes each history and attends in float64 "
                      f"(numpy); {done_bytes / 1e9:.3f} GB of the step's algorithmic bytes"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="b32-100k-g128", choices=sorted(workloads()))
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8, help="KV heads in the oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 2 GiB device copy (bandwidth reference, PMC scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path runs within one MI355X and "
              "launches no collectives; --gpus must be 1", file=sys.stderr)
        return 2

    import torch
    import bit_rotated_kv_split_amd as ok
    from bit_rotated_kv_split_amd import workload as W
    from bit_rotated_kv_split_amd.hipevents import HipEvent
    from bit_rotated_kv_split_amd.kvcache import DecodeWorkspace, Rotation
    from synth import gen

    torch.cuda.set_device(0)
    w = workloads()[args.workload]()
    steps, warmup = args.steps, args.warmup
    total = steps + warmup
    layout = W.Layout(w, None, extra_tokens=total)
    model = W.SyntheticModel(w)
    B, hq, hkv = w.batch, w.num_q_heads, w.num_kv_heads
    dims = ok.make_dims(hq, hkv, w.group_size)
    stream = torch.cuda.current_stream().cuda_stream

    # offline calibration, by the library
    t0 = time.perf_counter()
    qc, kc, vc = model.calibration()
    n_cal = qc.shape[0]
    cws = torch.empty(ok.oscar_calibrate_workspace_bytes(dims, n_cal), dtype=torch.uint8, device="cuda")
    r_k = torch.empty((hkv, 128, 128), dtype=torch.float32, device="cuda")
    r_v = torch.empty_like(r_k)
    c_k = torch.empty((hkv, 128), dtype=torch.float32, device="cuda")
    c_v = torch.empty_like(c_k)
    ok.oscar_calibrate(dims, n_cal, torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(),
                       torch.from_numpy(vc).cuda(), w.clip_pct, r_k, r_v, c_k, c_v, None, None, cws,
                       cws.numel())
    calib_s = time.perf_counter() - t0
    del cws
    rot = Rotation(r_k, r_v, c_k, c_v)

    t0 = time.perf_counter()
    cache = W.build_cache(w, layout, model, rot)
    fill_s = time.perf_counter() - t0

    # per-step inputs, resident before timing
    lens_all = layout.lens[None, :] + np.arange(1, total + 1)[:, None]
    seq_dev = torch.from_numpy(lens_all.astype(np.int32)).cuda()
    q_all = torch.stack([W.queries_tensor(model, s, B) for s in range(1, total + 1)])
    kn = np.zeros((total, B, hkv, 128), np.uint16)
    vn = np.zeros_like(kn)
    for b in range(B):
        p0 = int(layout.lens[b])
        for j in range(hkv):
            for src, a, n in layout.src_ranges(b, p0, total):
                kn[a - p0:a - p0 + n, b, j] = gen.kv_tokens_bf16(w.seed, "k", src, j, a, n, model.k_scale[j])
                vn[a - p0:a - p0 + n, b, j] = gen.kv_tokens_bf16(w.seed, "v", src, j, a, n, model.v_scale[j])
    kn_all = torch.from_numpy(kn.view(np.int16)).view(torch.bfloat16).cuda()
    vn_all = torch.from_numpy(vn.view(np.int16)).view(torch.bfloat16).cuda()
    max_len = int(lens_all.max())
    ws = DecodeWorkspace(dims, B, max_len)
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    base = cache.struct()
    structs = [ok.make_cache(cache.pages, cache.n_pages, cache.sink_k, cache.sink_v, cache.recent_k,
                             cache.recent_v, cache.page_table, cache.max_pages_per_req,
                             seq_dev[s].data_ptr(), B) for s in range(total)]
    del base
    kind = {"auto": 0, "valu": 1, "mfma": 2}[args.kernel]
    ok.oscar_set_history_kernel(kind)
    ev_b = [HipEvent() for _ in range(steps)]
    ev_a = [HipEvent() for _ in range(steps)]

    def step(s: int, timed_idx: int | None):
        c = structs[s]
        if timed_idx is None:
            ok.oscar_set_history_events(None, None)
        else:
            ok.oscar_set_history_events(ev_b[timed_idx].ptr, ev_a[timed_idx].ptr)
        ok.oscar_decode_step(dims, rot.struct, c, kn_all[s], vn_all[s], q_all[s], max_len, ws.buf,
                             ws.nbytes, out, None, stream)

    for s in range(warmup):
        step(s, None)
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: B={B} Hq={hq} Hkv={hkv} G={w.group_size} L0={int(layout.lens.min())}.."
          f"{int(layout.lens.max())} splits={ws.splits} calib {calib_s:.1f}s fill {fill_s:.1f}s",
          file=sys.stderr, flush=True)
    start, end = HipEvent(), HipEvent()
    start.record(stream)
    for i in range(steps):
        step(warmup + i, i)
    end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    ok.oscar_set_history_events(None, None)
    step_ms = start.elapsed_ms(end) / steps
    k3_ms = [ev_b[i].elapsed_ms(ev_a[i]) for i in range(steps)]

    kname = "mfma" if ok.oscar_history_kernel_for(dims) == 2 else "valu"
    # the timed launch: history splits, plus the bf16 sink/recent chunks when
    # the matrix-core kernel runs them in the same launch
    launch_tot = 0
    step_tot = 0
    for i in range(steps):
        lens_i = lens_all[warmup + i]
        hb, sb = step_bytes(lens_i, hkv, hq, w.group_size)
        launch_tot += hb + (bf16_bytes(lens_i, hkv) if kname == "mfma" else 0)
        step_tot += sb
    k3_gbs = launch_tot / (sum(k3_ms) * 1e-3) / 1e9
    value = step_tot / (step_ms * 1e-3 * steps) / 1e9
    traffic = load_traffic(args.workload, kname)

    copy_gbs = None
    if args.copy_probe:
        nb = 2 << 30
        src = torch.empty(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        c0, c1 = HipEvent(), HipEvent()
        c0.record(stream)
        dst.copy_(src)
        c1.record(stream)
        c1.synchronize()
        copy_gbs = round(2 * nb / (c0.elapsed_ms(c1) * 1e-3) / 1e9, 1)
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        hosted = {"r_k32": r_k.cpu().numpy(), "r_v32": r_v.cpu().numpy(),
                  "clip_k": c_k.cpu().numpy(), "clip_v": c_v.cpu().numpy()}
        cpu = cpu_baseline(model, layout, hosted, lens_all[-1], min(args.cpu_heads, hkv))

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(step_ms, 4),
        "us_per_step": round(step_ms * 1e3, 2),
        "pct_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2+bf16 storage, f32 accumulate",
        "data": "synthetic (seeded generator; library-calibrated rotations)",
        "config": {"workload": w.name, "batch": B, "context": int(layout.lens.max()),
                   "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128,
                   "group_size": w.group_size, "page_size": 64, "history_splits": ws.splits,
                   "history_kernel": kname, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(k3_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(k3_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": f"history ({kname})" + (" + bf16 sink/recent" if kname == "mfma" else ""),
                     "avg_us": round(1e3 * sum(k3_ms) / steps, 2),
                     "bytes_per_launch": int(launch_tot / steps),
                     "unit_bytes": {"history_token_head": hist_unit_bytes(w.group_size),
                                    "bf16_token_head": 512}},
        "cpu_baseline": cpu,
        "copy_gbs": copy_gbs,
        "calibration_s": round(calib_s, 2),
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
