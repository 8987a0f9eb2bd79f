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
PAGE = 64
METRIC = "decode-attn µs/step + achieved HBM GB/s (% peak), 100K ctx, batch 32"


def workloads():
    import dataclasses
    from synth import configs, gen
    return {
        "b32-100k-g128": lambda: configs.qwen3_8b_b32(128),
        "b32-100k-g64": lambda: configs.qwen3_8b_b32(64),
        "b32-100k-g32": lambda: configs.qwen3_8b_b32(32),
        "b32-100k-g128-lloyd": lambda: dataclasses.replace(configs.qwen3_8b_b32(128),
                                                           name="qwen3-8b-b32-100k-lloyd-max", codebook=1),
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


def _host_cpu():
    """CPU model name and logical core count of this host."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count() or 1


def cpu_baseline(model, layout, cal_host, lens, n_heads: int, budget_s: float = 10.0,
                 single_budget_s: float = 4.0):
    """Time the oracle (as it stands) on whole requests of the same workload
    at their final length, request 0 first, until about budget_s seconds of
    oracle work with numpy's default threads, then again single-threaded
    (BLAS limited to one thread) for about single_budget_s; each scaled to
    GB/s of the same algorithmic bytes.  The sample's tokens come from the GPU
    twin of the seeded generator (bit-identical to synth.gen; not timed)."""
    import torch
    from oracle import oscar as O
    from synth import gpu as synth_gpu
    w = model.w
    g = w.gqa
    stream = torch.cuda.current_stream().cuda_stream
    codebook = ("uniform", "lloyd-max")[w.codebook]

    def request_inputs(b):
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
        return L, host

    def run(budget, heads):
        spent, done_bytes, reqs = 0.0, 0, 0
        for b in range(w.batch):
            L, host = request_inputs(b)
            q = model.queries(0, w.batch)[b][: heads * g]
            t0 = time.perf_counter()
            O.request_attention(q, host["k"][:, :heads], host["v"][:, :heads], cal_host["r_k32"][:heads],
                                cal_host["r_v32"][:heads], cal_host["clip_k"][:heads], cal_host["clip_v"][:heads],
                                w.group_size, codebook)
            spent += time.perf_counter() - t0
            done_bytes += step_bytes(np.array([L]), heads, heads * g, w.group_size)[1]
            reqs += 1
            if spent >= budget:
                break
        return spent, done_bytes, reqs

    spent, done_bytes, reqs = run(budget_s, n_heads)
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
        with threadpool_limits(limits=1):
            s1, b1, r1 = run(single_budget_s, 1)
        single = {"value": round(b1 / s1 / 1e9, 4), "seconds": round(s1, 3),
                  "sample": f"requests 0..{r1 - 1}, KV head 0 only, one thread"}
    except Exception:
        cores, single = 1, None
    cpu_model, nproc = _host_cpu()
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seconds": round(spent, 3),
            "sample": f"requests 0..{reqs - 1} of {w.batch}, {n_heads} of {w.num_kv_heads} KV heads each, "
                      f"at their final lengths: the oracle demotes each history and attends in float64 "
                      f"(numpy); {done_bytes / 1e9:.3f} GB of the step's algorithmic bytes",
            "single_thread": single, "host_cpu": cpu_model, "host_logical_cores": nproc}


def default_layers(workload: str) -> int:
    """Independent layer caches a run cycles through: the single-request
    workload's cache (57 MB) would otherwise sit in the 256 MB last-level
    cache, so ten are cycled (one per step) to keep its reads in HBM."""
    return 10 if workload == "b1-100k" else 1


def pct(xs, q):
    return round(float(np.percentile(np.asarray(xs), q)), 2)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (0: the workload's own count, 100 for b1-100k and 200 for "
                         "b32-ragged-gqa8, else 100)")
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first (the GPU's clocks settle over the first tens of steps)")
    ap.add_argument("--workload", default="b32-100k-g128", choices=sorted(workloads()))
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--layers", type=int, default=0,
                    help="independent layer caches cycled one per step (0: 10 for b1-100k, else 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8, help="KV heads in the oracle sample")
    ap.add_argument("--bf16-baseline", choices=["auto", "on", "off"], default="auto",
                    help="also time the all-bf16 cache decode step (auto: on for the 32 x 100K workloads)")
    ap.add_argument("--history-target", type=int, default=0,
                    help="history workgroups the split schedule aims for (0: the library default)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="accepted for older command lines; the 2 GiB copy probe always runs")
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
    steps, warmup = args.steps or (w.steps if w.steps > 1 else 100), args.warmup
    total = steps + warmup
    n_layers = args.layers or default_layers(args.workload)
    appends = -(-total // n_layers)          # tokens each layer cache receives
    layout = W.Layout(w, None, extra_tokens=appends)
    model = W.SyntheticModel(w)
    B, hq, hkv = w.batch, w.num_q_heads, w.num_kv_heads
    dims = ok.make_dims(hq, hkv, w.group_size, codebook=w.codebook)
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
    caches = [W.build_cache(w, layout, model, rot) for _ in range(n_layers)]
    fill_s = time.perf_counter() - t0

    # per-step inputs, resident before timing.  Step s runs layer s % n_layers
    # after that layer's (s // n_layers + 1)-th append.
    lens_t = layout.lens[None, :] + np.arange(1, appends + 1)[:, None]      # [appends][B]
    lens_step = np.stack([lens_t[s // n_layers] for s in range(total)])
    seq_dev = torch.from_numpy(lens_t.astype(np.int32)).cuda()
    q_all = torch.stack([W.queries_tensor(model, s, B) for s in range(1, total + 1)])
    kn = np.zeros((appends, B, hkv, 128), np.uint16)
    vn = np.zeros_like(kn)
    for b in range(B):
        p0 = int(layout.lens[b])
        for j in range(hkv):
            for src, a, n in layout.src_ranges(b, p0, appends):
                kn[a - p0:a - p0 + n, b, j] = gen.kv_tokens_bf16(w.seed, "k", src, j, a, n, model.k_scale[j])
                vn[a - p0:a - p0 + n, b, j] = gen.kv_tokens_bf16(w.seed, "v", src, j, a, n, model.v_scale[j])
    kn_all = torch.from_numpy(kn.view(np.int16)).view(torch.bfloat16).cuda()
    vn_all = torch.from_numpy(vn.view(np.int16)).view(torch.bfloat16).cuda()
    max_len = int(lens_t.max())
    ok.oscar_set_history_target(args.history_target)
    ws = DecodeWorkspace(dims, B, max_len)
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    structs = [[ok.make_cache(c.pages, c.n_pages, c.sink_k, c.sink_v, c.recent_k, c.recent_v, c.page_table,
                              c.max_pages_per_req, seq_dev[t].data_ptr(), B) for t in range(appends)]
               for c in caches]
    kind = {"auto": 0, "valu": 1, "mfma": 2}[args.kernel]
    ok.oscar_set_history_kernel(kind)

    def timed_run(one_step):
        """Warm up, then time `steps` steps: per-step and history-launch events."""
        ev_b = [HipEvent() for _ in range(steps)]
        ev_a = [HipEvent() for _ in range(steps)]
        marks = [HipEvent() for _ in range(steps + 1)]
        for s in range(warmup):
            ok.oscar_set_history_events(None, None)
            one_step(s)
        torch.cuda.synchronize()
        for i in range(steps):
            marks[i].record(stream)
            ok.oscar_set_history_events(ev_b[i].ptr, ev_a[i].ptr)
            one_step(warmup + i)
        marks[steps].record(stream)
        marks[steps].synchronize()
        torch.cuda.synchronize()
        ok.oscar_set_history_events(None, None)
        step_us = [1e3 * marks[i].elapsed_ms(marks[i + 1]) for i in range(steps)]
        hist_us = [1e3 * ev_b[i].elapsed_ms(ev_a[i]) for i in range(steps)]
        return step_us, hist_us

    def int2_step(s: int):
        t = s // n_layers
        ok.oscar_decode_step(dims, rot.struct, structs[s % n_layers][t], kn_all[t], vn_all[t], q_all[s], max_len,
                             ws.buf, ws.nbytes, out, None, stream)

    print(f"[bench] {w.name}: B={B} Hq={hq} Hkv={hkv} G={w.group_size} L0={int(layout.lens.min())}.."
          f"{int(layout.lens.max())} layers={n_layers} slots={ws.splits} calib {calib_s:.1f}s fill {fill_s:.1f}s",
          file=sys.stderr, flush=True)
    step_us, k3_us = timed_run(int2_step)
    step_ms = sum(step_us) / steps / 1e3

    kname = "mfma" if ok.oscar_history_kernel_for(dims) == 2 else "valu"
    # the timed launch: history splits, plus the bf16 sink/recent chunks when
    # the matrix-core kernel runs them in the same launch
    launch_tot = 0
    step_tot = 0
    unique_tot = 0
    for i in range(steps):
        lens_i = lens_step[warmup + i]
        hb, sb = step_bytes(lens_i, hkv, hq, w.group_size)
        launch_tot += hb + (bf16_bytes(lens_i, hkv) if kname == "mfma" else 0)
        step_tot += sb
        shared_tok = PAGE * (sum(layout.shared_pages) - layout.chain_len) if layout.chain_len else 0
        unique_tot += sb - shared_tok * hkv * hist_unit_bytes(w.group_size)
    k3_gbs = launch_tot / (sum(k3_us) * 1e-6) / 1e9
    value = step_tot / (sum(step_us) * 1e-6) / 1e9
    traffic = load_traffic(args.workload, kname)

    # bandwidth reference: one 2 GiB device copy
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

    base = None
    if args.bf16_baseline == "on" or (args.bf16_baseline == "auto" and args.workload in ("b32-100k-g128",
                                                                                       "b32-100k-g64")):
        base = bf16_baseline(ok, W, HipEvent, torch, w, layout, lens_t, appends, q_all, kn_all, vn_all, max_len,
                             timed_run, n_layers, stream, dims, hkv, hq)
        if base is not None:
            base["int2_step_speedup"] = round(base["us_per_step"] / (step_ms * 1e3), 3)
            base["int2_history_speedup"] = round(base["history_us"] / (sum(k3_us) / steps), 3)
            base["byte_ratio"] = round(base["bytes_per_step"] / (step_tot / steps), 3)

    cpu = None
    if not args.no_cpu_baseline:
        hosted = {"r_k32": r_k.cpu().numpy(), "r_v32": r_v.cpu().numpy(),
                  "clip_k": c_k.cpu().numpy(), "clip_v": c_v.cpu().numpy()}
        cpu = cpu_baseline(model, layout, hosted, lens_step[-1], min(args.cpu_heads, hkv))

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(step_ms, 4),
        "us_per_step": round(step_ms * 1e3, 2),
        "step_us_p50": pct(step_us, 50),
        "step_us_p99": pct(step_us, 99),
        "pct_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic: int8 x int8 -> int32 matrix-core products (query and
        # softmax-weight digits against 2-bit codes) and float32 softmax,
        # scales and accumulation; the cache holds 2-bit codes and bf16
        "dtype": "i8-mfma+f32" if kname == "mfma" else "f32",
        "storage": "int2 history (bf16 scale/zero) + bf16 sink/recent",
        "data": "synthetic (seeded generator; library-calibrated rotations)",
        "config": {"workload": w.name, "batch": B, "context": int(layout.lens.max()),
                   "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128,
                   "group_size": w.group_size, "codebook": ("uniform", "lloyd-max")[w.codebook],
                   "page_size": 64, "history_split_slots": ws.splits, "history_target": args.history_target,
                   "layer_caches": n_layers, "history_kernel": kname, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(k3_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(k3_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": f"history ({kname})" + (" + bf16 sink/recent" if kname == "mfma" else ""),
                     "avg_us": round(sum(k3_us) / steps, 2),
                     "bytes_per_launch": int(launch_tot / steps),
                     "frac_of_copy": round(k3_gbs / copy_gbs, 4),
                     "unit_bytes": {"history_token_head": hist_unit_bytes(w.group_size),
                                    "bf16_token_head": 512}},
        "copy_gbs": copy_gbs,
        "cpu_baseline": cpu,
        "bf16_baseline": base,
        "calibration_s": round(calib_s, 2),
    }
    if layout.chain_len:
        res["unique_value"] = round(unique_tot / (sum(step_us) * 1e-6) / 1e9, 2)
    print(json.dumps(res), flush=True)
    return 0


def bf16_baseline(ok, W, HipEvent, torch, w, layout, lens_t, appends, q_all, kn_all, vn_all, max_len, timed_run,
                  n_layers, stream, dims, hkv, hq):
    """The same steps on an all-bf16 cache (oscar_bf16_append + oscar_bf16_decode)."""
    if n_layers != 1:
        return None
    t0 = time.perf_counter()
    bcache = W.build_bf16_cache(w, layout, extra_tokens=appends)
    fill_s = time.perf_counter() - t0
    seq_dev = torch.from_numpy(lens_t.astype(np.int32)).cuda()
    structs = [ok.make_bf16_cache(bcache.pages, bcache.n_pages, bcache.page_table, bcache.max_pages_per_req,
                                  seq_dev[t].data_ptr(), w.batch) for t in range(appends)]
    nb = ok.oscar_bf16_decode_workspace_bytes(dims, w.batch)
    wsb = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, hq, 128), dtype=torch.float32, device="cuda")

    def one(s: int):
        ok.oscar_bf16_append(dims, structs[s], kn_all[s], vn_all[s], stream)
        ok.oscar_bf16_decode(dims, structs[s], q_all[s], max_len, wsb, nb, out, None, stream)

    step_us, hist_us = timed_run(one)
    steps = len(step_us)
    warm = len(lens_t) - steps
    hist_b = [int(lens_t[warm + i].sum()) * hkv * 512 for i in range(steps)]
    step_b = [hb + w.batch * hq * 128 * (2 + 4) + w.batch * hkv * 512 for hb in hist_b]
    del bcache, wsb
    torch.cuda.empty_cache()
    h_gbs = sum(hist_b) / (sum(hist_us) * 1e-6) / 1e9
    return {"us_per_step": round(sum(step_us) / steps, 2), "step_us_p50": pct(step_us, 50),
            "value": round(sum(step_b) / (sum(step_us) * 1e-6) / 1e9, 2), "unit": "GB/s",
            "history_us": round(sum(hist_us) / steps, 2), "history_gbs": round(h_gbs, 1),
            "history_frac": round(h_gbs / PEAK_HBM_GBS, 4), "bytes_per_step": int(sum(step_b) / steps),
            "fill_s": round(fill_s, 1),
            "what": "oscar_bf16_append + oscar_bf16_decode over the same tokens, all in bf16 pages"}


if __name__ == "__main__":
    sys.exit(main())
