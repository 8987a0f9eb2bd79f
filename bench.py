#!/usr/bin/env python3
"""Decode-step benchmark of the OSCAR INT2 KV-cache path on one MI355X.

A step is one pass of the whole hot path over the batch (oscar_decode_step):
append + demotion, query rotation and the split schedule in one launch; INT2
history split-K + bf16 sink/recent in a second; LSE merge + value
un-rotation in a third.  Inputs (cache, queries, new tokens, lengths) are
resident in HBM before timing starts; every step appends one token per
request, so lengths grow by one.

Default workload: 32 requests at 100K context, 32 query / 8 KV heads,
head_dim 128, G = 128, paged cache (64-token pages, seeded random page
permutation), synthetic seeded data; rotations and clips calibrated by the
library from a synthetic calibration sequence before timing.

Order of one run:
  1. calibration, cache fill, per-step inputs (untimed);
  2. bandwidth probes: streaming HBM reads (grid-stride non-temporal and
     plain loads, and 4 KB blocks read front to back by one-wave
     workgroups, the history kernel's access pattern) repeated for about
     0.3 s, and a 2 GiB copy.  They give the read ceiling the roofline is
     compared against, and they leave the GPU at its steady clocks, so the
     timed steps do not measure the clock ramp that follows the idle setup;
  3. `warmup` untimed steps, then exactly `steps` timed steps between one
     pair of events: `value` and `ms_per_step`; every 4th of their history
     launches (`--launch-event-every`) between its own events (`roofline`,
     per-quarter means; an event pair adds about 4 us to its step, so not
     every step carries one), and the shader clock over every launch; then
     `steps` more steps with an event between consecutive steps for the
     per-step latency (`step_us_p50`, `step_us_p99`);
  4. `cold_start`: after 1 s with the GPU idle, 20 more timed steps with no
     warm-up (diagnostic: the cost of starting from idle clocks);
  5. the all-bf16 baseline's steps (the 32 x 100K workloads);
  6. the oracle on the host cores (`cpu_baseline`): the plain C++ oracle
     on OpenMP threads, and the numpy oracle in worker processes started
     before the GPU is touched.

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
COLD_STEPS = 20
COLD_IDLE_S = 1.0


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


# ----------------------------------------------------------------------------
# CPU baseline: the oracle in worker processes (one BLAS thread each)

def _oracle_worker(conn) -> None:
    """Body of one oracle worker process.  Receives ("task", args) messages
    (the arguments of oracle.request_attention for one (request, KV head)
    pair, plus its algorithmic bytes), holds them until ("go",), then runs
    them back to back and replies (start, end, bytes, count) on the
    system-wide monotonic clock; ("stop",) ends the process."""
    from threadpoolctl import threadpool_limits
    from oracle import oscar as O
    tasks = []
    with threadpool_limits(limits=1):
        while True:
            msg = conn.recv()
            if msg[0] == "task":
                tasks.append(msg[1])
            elif msg[0] == "go":
                t0 = time.monotonic()
                nbytes = 0
                for args, nb in tasks:
                    O.request_attention(*args)
                    nbytes += nb
                t1 = time.monotonic()
                conn.send((t0, t1, nbytes, len(tasks)))
                tasks = []
            else:
                break


class OracleWorkers:
    """Worker processes for the oracle's CPU baseline.  They are started
    (spawned, with one-thread BLAS in their environment) before this process
    touches the GPU, and only ever run numpy."""

    def __init__(self, n: int):
        import multiprocessing as mp
        ctx = mp.get_context("spawn")
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        for k in saved:
            os.environ[k] = "1"
        self.conns, self.procs = [], []
        try:
            for _ in range(n):
                a, b = ctx.Pipe()
                p = ctx.Process(target=_oracle_worker, args=(b,), daemon=True)
                p.start()
                self.conns.append(a)
                self.procs.append(p)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def run(self, assignments):
        """assignments[w] = list of (args, bytes) for worker w; all workers
        start together.  Returns (bytes, wall seconds, per-worker busy seconds)."""
        used = [w for w, tasks in enumerate(assignments) if tasks]
        for w in used:
            for t in assignments[w]:
                self.conns[w].send(("task", t))
        for w in used:
            self.conns[w].send(("go",))
        res = [self.conns[w].recv() for w in used]
        wall = max(r[1] for r in res) - min(r[0] for r in res)
        return sum(r[2] for r in res), wall, [r[1] - r[0] for r in res]

    def close(self):
        for c in self.conns:
            try:
                c.send(("stop",))
            except (OSError, BrokenPipeError):
                pass
        for p in self.procs:
            p.join(timeout=10)


def cpu_baseline(workers: OracleWorkers, model, layout, cal_host, lens, cpp_requests: int = 4,
                 cpp_single_pairs: int = 3, numpy_requests: int = 2):
    """The oracle (as it stands) on the host cores, at the workload's final
    lengths, one (request, KV head) pair per task: demote the pair's history
    and attend in float64.  `value` is the plain C++ oracle
    (oracle/oscar_ref.cpp) with OpenMP threads over the pairs of requests
    0 .. cpp_requests-1 (every KV head), as many threads as this process's
    CPU share (at most 16); `single_thread` runs `cpp_single_pairs` pairs (KV
    head 0 of successive requests) on one thread.  `numpy_oracle` is the
    numpy oracle (BLAS products) over the pairs of numpy_requests requests
    in the worker processes, one BLAS thread each.  Every leg is scaled to
    GB/s of the same algorithmic bytes.  The pairs' tokens come from the GPU
    twin of the seeded generator (bit-identical to synth.gen; not timed)."""
    import torch
    from oracle import cpp as C
    from synth import gpu as synth_gpu
    w = model.w
    g, hkv = w.gqa, w.num_kv_heads
    stream = torch.cuda.current_stream().cuda_stream
    codebook = ("uniform", "lloyd-max")[w.codebook]
    q_all = model.queries(0, w.batch)
    fetched = {}

    def tokens(b):
        """Host bf16 bits [L][Hkv][128] of request b's K and V tokens."""
        if b not in fetched:
            L = int(lens[b])
            host = {}
            for which, scale in (("k", model.k_scale), ("v", model.v_scale)):
                buf = torch.empty((L, hkv, 128), dtype=torch.int16, device="cuda")
                sc = torch.from_numpy(np.ascontiguousarray(scale)).cuda()
                for src, p0, n in layout.src_ranges(b, 0, L):
                    synth_gpu.fill_kv(buf.data_ptr() + 2 * p0 * hkv * 128, n, hkv, hkv * 128, 128,
                                      w.seed, which, src, p0, sc, stream)
                torch.cuda.synchronize()
                host[which] = buf.cpu().numpy().view(np.uint16)
                del buf
            fetched[b] = host
        return fetched[b]

    def pair_bytes(b):
        return step_bytes(np.array([int(lens[b])]), 1, g, w.group_size)[1]

    def cpp_pairs(b, heads):
        h = tokens(b)
        L = h["k"].shape[0]
        k, v = h["k"].reshape(L, hkv * 128), h["v"].reshape(L, hkv * 128)
        return [{"q": q_all[b][j * g:(j + 1) * g], "k": k, "v": v, "off": j * 128,
                 "r_k": cal_host["r_k32"][j], "r_v": cal_host["r_v32"][j],
                 "clip_k": cal_host["clip_k"][j], "clip_v": cal_host["clip_v"][j]} for j in heads]

    def numpy_tasks(b):
        h = tokens(b)
        return [((q_all[b][j * g:(j + 1) * g], np.ascontiguousarray(h["k"][:, j:j + 1]),
                  np.ascontiguousarray(h["v"][:, j:j + 1]), cal_host["r_k32"][j:j + 1],
                  cal_host["r_v32"][j:j + 1], cal_host["clip_k"][j:j + 1], cal_host["clip_v"][j:j + 1],
                  w.group_size, codebook), pair_bytes(b)) for j in range(hkv)]

    threads = cpu_worker_count()
    reqs = list(range(min(cpp_requests, w.batch)))
    par = [p for b in reqs for p in cpp_pairs(b, range(hkv))]
    par_bytes = sum(pair_bytes(b) * hkv for b in reqs)
    C.lib()
    t0 = time.perf_counter()
    C.attend_pairs(par, g, w.group_size, codebook, threads)
    par_wall = time.perf_counter() - t0
    singles = list(range(min(cpp_single_pairs, w.batch)))
    one = [p for b in singles for p in cpp_pairs(b, [0])]
    one_bytes = sum(pair_bytes(b) for b in singles)
    t0 = time.perf_counter()
    C.attend_pairs(one, g, w.group_size, codebook, 1)
    one_wall = time.perf_counter() - t0

    n = len(workers.conns)
    np_reqs = list(range(min(numpy_requests, w.batch)))
    tasks = [t for b in np_reqs for t in numpy_tasks(b)]
    np_bytes, np_wall, busy = workers.run([tasks[i::n] for i in range(n)])
    cpu_model, nproc = _host_cpu()
    return {"value": round(par_bytes / par_wall / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(par_wall, 3),
            "sample": f"{len(par)} (request, KV head) pairs: requests 0..{reqs[-1]} of {w.batch}, all {hkv} KV "
                      f"heads, at their final lengths; each pair's history demoted and attended in float64 by "
                      f"the plain C++ oracle, {threads} OpenMP threads over the pairs, "
                      f"{par_bytes / 1e9:.3f} GB of the step's algorithmic bytes",
            "single_thread": {"value": round(one_bytes / one_wall / 1e9, 4), "seconds": round(one_wall, 3),
                              "sample": f"{len(one)} pairs (KV head 0 of requests 0..{singles[-1]}), "
                                        f"C++ oracle, one thread"},
            "parallel_speedup": round((par_bytes / par_wall) / (one_bytes / one_wall), 2),
            "numpy_oracle": {"value": round(np_bytes / np_wall / 1e9, 4), "cores": n,
                             "seconds": round(np_wall, 3),
                             "sample": f"{len(tasks)} pairs (requests 0..{np_reqs[-1]}, all KV heads), numpy "
                                       f"oracle, {n} worker processes with one BLAS thread each",
                             "worker_busy_s": [round(x, 3) for x in busy]},
            "host_cpu": cpu_model, "host_logical_cores": nproc}


def cpu_worker_count() -> int:
    """OpenMP threads and worker processes of the oracle baseline: this
    process's CPU share, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------

def default_layers(workload: str) -> int:
    """Independent layer caches a run cycles through: the single-request
    workload's cache (57 MB) would otherwise sit in the 256 MB last-level
    cache, so ten are cycled (one per step) to keep its reads in HBM."""
    return 10 if workload == "b1-100k" else 1


def pct(xs, q):
    return round(float(np.percentile(np.asarray(xs), q)), 2)


def quarters(xs):
    """Means of the first and the last quarter of a sequence of timings."""
    xs = np.asarray(xs, dtype=np.float64)
    k = max(1, len(xs) // 4)
    return [round(float(xs[:k].mean()), 2), round(float(xs[-k:].mean()), 2)]


def bandwidth_probes(ok, torch, HipEvent, stream, settle_s: float = 0.3, nbytes: int = 4 << 30):
    """HBM read ceiling: the library's read probes over nbytes (grid-stride
    16-byte loads, non-temporal and plain, and the block-streaming probe,
    2048 one-wave workgroups reading 4 KB blocks front to back with
    non-temporal loads, the history kernel's access pattern), alternated for
    about settle_s seconds; median GB/s of the second half of each kind's
    passes; the ceiling is the fastest kind.  Also a device copy of nbytes /
    2 (read + write bytes / time, median of 5; the 2 GiB copy the traffic
    counters are scaled by)."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    kinds = {"read_nontemporal_gbs": lambda: ok.oscar_probe_read(buf, nbytes, True, sink, stream),
             "read_plain_gbs": lambda: ok.oscar_probe_read(buf, nbytes, False, sink, stream),
             "read_blocks_gbs": lambda: ok.oscar_probe_read_blocks(buf, nbytes, True, 2048, sink, stream)}
    times = {k: [] for k in kinds}
    t_end = time.perf_counter() + settle_s
    e0, e1 = HipEvent(), HipEvent()
    while time.perf_counter() < t_end or min(len(v) for v in times.values()) < 6:
        for k, run in kinds.items():
            e0.record(stream)
            run()
            e1.record(stream)
            e1.synchronize()
            times[k].append(e0.elapsed_ms(e1))
    rates = {}
    for k, ts in times.items():
        ts = ts[len(ts) // 2:]
        rates[k] = nbytes / (float(np.median(ts)) * 1e-3) / 1e9
    half = nbytes // 2
    src, dst = buf[:half], buf[half:]
    copies = []
    for _ in range(5):
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        e1.synchronize()
        copies.append(e0.elapsed_ms(e1))
    copy_gbs = 2 * half / (float(np.median(copies)) * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    res = {k: round(v, 1) for k, v in rates.items()}
    res.update(read_ceiling_gbs=round(max(rates.values()), 1), copy_gbs=round(copy_gbs, 1),
               passes=sum(len(v) for v in times.values()), buffer_bytes=nbytes)
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (0: the workload's own count, 100 for b1-100k and 200 for "
                         "b32-ragged-gqa8, else 100)")
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps before the timed ones")
    ap.add_argument("--workload", default="b32-100k-g128", choices=sorted(workloads()))
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--layers", type=int, default=0,
                    help="independent layer caches cycled one per step (0: 10 for b1-100k, else 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold-start", action="store_true", help="skip the idle-start diagnostic leg")
    ap.add_argument("--launch-event-every", type=int, default=4,
                    help="time every n-th history launch of the timed steps between its own HIP events "
                         "(an event pair adds about 4 us to its step; 1 = every launch)")
    ap.add_argument("--bf16-baseline", choices=["auto", "on", "off"], default="auto",
                    help="also time the all-bf16 cache decode step (auto: on for the 32 x 100K workloads)")
    ap.add_argument("--history-target", type=int, default=0,
                    help="history workgroups the split schedule aims for (0: the library default)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="accepted for older command lines; the probes always run")
    ap.add_argument("--trace-file", default="",
                    help="also write every timed step's step and history-launch times (µs) to this JSON file")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path runs within one MI355X and "
              "launches no collectives; --gpus must be 1", file=sys.stderr)
        return 2

    # the oracle's worker processes start before anything touches the GPU
    workers = None if args.no_cpu_baseline else OracleWorkers(cpu_worker_count())

    import torch
    import bit_rotated_kv_split_amd as ok
    from bit_rotated_kv_split_amd import workload as W
    from bit_rotated_kv_split_amd.hipevents import HipEvent
    from bit_rotated_kv_split_amd.kvcache import DecodeWorkspace, Rotation
    from synth import gen

    torch.cuda.set_device(0)
    w = workloads()[args.workload]()
    steps, warmup = args.steps or (w.steps if w.steps > 1 else 100), args.warmup
    n_cold = 0 if args.no_cold_start else COLD_STEPS
    total = warmup + 2 * steps + n_cold     # warm-up, timed, latency leg, cold start
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
    kind = {"auto": 0, "valu": 1, "mfma": 2}[args.kernel]
    base_opts = ok.make_options(history_kernel=kind, history_target=args.history_target)
    ws = DecodeWorkspace(dims, B, max_len, options=base_opts)
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    structs = [[ok.make_cache(c.pages, c.n_pages, c.sink_k, c.sink_v, c.recent_k, c.recent_v, c.page_table,
                              c.max_pages_per_req, seq_dev[t].data_ptr(), B) for t in range(appends)]
               for c in caches]

    wall_khz = ok.wall_clock_khz()

    def timed_run(one_step, first: int, n_warm: int, n_timed: int, marks_per_step: bool = False,
                  event_every: int = 1):
        """Steps first .. first+n_warm-1 untimed, then n_timed steps timed
        between one pair of events on the stream.  Timed step i's history
        launch runs between its own start/stop events (hipExtLaunchKernelGGL)
        when event_every > 0 and i % event_every == 0 (an event pair adds
        about 4 µs to its step, so the headline steps time only a sample of
        launches), and every launch records the shader clock over its first
        workgroup (free).  With marks_per_step an event is also recorded
        between consecutive steps (per-step times, at a few µs of extra cost
        per step).  Returns (total µs, per-step µs or None, the timed
        launches' indices and µs, per-launch MHz of every timed launch)."""
        ev_b = [HipEvent() for _ in range(n_timed)]
        ev_a = [HipEvent() for _ in range(n_timed)]
        marks = [HipEvent() for _ in range(n_timed + 1)]
        clk = torch.zeros((n_timed, 4), dtype=torch.int64, device="cuda")
        timed = [i for i in range(n_timed) if event_every > 0 and i % event_every == 0]
        opts = [ok.make_options(kind, args.history_target, ev_b[i], ev_a[i], clk.data_ptr() + 32 * i)
                if i in timed else ok.make_options(kind, args.history_target, None, None, clk.data_ptr() + 32 * i)
                for i in range(n_timed)]
        for s in range(n_warm):
            one_step(first + s, base_opts)
        torch.cuda.synchronize()
        marks[0].record(stream)
        for i in range(n_timed):
            if marks_per_step and i > 0:
                marks[i].record(stream)
            one_step(first + n_warm + i, opts[i])
        marks[n_timed].record(stream)
        marks[n_timed].synchronize()
        torch.cuda.synchronize()
        total_us = 1e3 * marks[0].elapsed_ms(marks[n_timed])
        step_us = [1e3 * marks[i].elapsed_ms(marks[i + 1]) for i in range(n_timed)] if marks_per_step else None
        hist_us = [1e3 * ev_b[i].elapsed_ms(ev_a[i]) for i in timed]
        c = clk.cpu().numpy().astype(np.float64)
        mhz = ((c[:, 2] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 1], 1) * wall_khz / 1e3).tolist()
        return total_us, step_us, (timed, hist_us), mhz

    def int2_step(s: int, opts):
        t = s // n_layers
        ok.oscar_decode_step(dims, rot.struct, structs[s % n_layers][t], kn_all[t], vn_all[t], q_all[s], max_len,
                             ws.buf, ws.nbytes, out, None, stream, options=opts)

    print(f"[bench] {w.name}: B={B} Hq={hq} Hkv={hkv} G={w.group_size} L0={int(layout.lens.min())}.."
          f"{int(layout.lens.max())} layers={n_layers} slots={ws.splits} calib {calib_s:.1f}s fill {fill_s:.1f}s",
          file=sys.stderr, flush=True)
    probes = bandwidth_probes(ok, torch, HipEvent, stream)
    every = max(1, args.launch_event_every)
    total_us, _, (k3_idx, k3_us), k3_mhz = timed_run(int2_step, 0, warmup, steps, event_every=every)
    step_ms = total_us / steps / 1e3
    # per-step latency: the next `steps` steps with an event between steps
    # (and none around the history launches)
    _, step_us, _, _ = timed_run(int2_step, warmup + steps, 0, steps, marks_per_step=True, event_every=0)

    kname = "mfma" if ok.oscar_history_kernel_for(dims, base_opts) == 2 else "valu"
    shared_tok = PAGE * (sum(layout.shared_pages) - layout.chain_len) if layout.chain_len else 0

    def byte_totals(first: int, n: int, only=None):
        """(history launch bytes, step bytes, unique step bytes) summed over
        steps first .. first+n-1 (or first + i for i in `only`): the launch
        holds the history splits, plus the bf16 sink/recent chunks when the
        matrix-core kernel runs them."""
        launch = stp = uniq = 0
        for i in (range(n) if only is None else only):
            lens_i = lens_step[first + i]
            hb, sb = step_bytes(lens_i, hkv, hq, w.group_size)
            launch += hb + (bf16_bytes(lens_i, hkv) if kname == "mfma" else 0)
            stp += sb
            uniq += sb - shared_tok * hkv * hist_unit_bytes(w.group_size)
        return launch, stp, uniq

    _, step_tot, unique_tot = byte_totals(warmup, steps)
    launch_tot, _, _ = byte_totals(warmup, steps, only=k3_idx)     # the launches timed by events
    k3_gbs = launch_tot / (sum(k3_us) * 1e-6) / 1e9
    k3_avg = sum(k3_us) / len(k3_us)
    value = step_tot / (total_us * 1e-6) / 1e9
    traffic = load_traffic(args.workload, kname)

    trace = {"history_us": k3_us, "history_mhz": k3_mhz, "latency_step_us": step_us}
    cold = None
    if n_cold:
        torch.cuda.synchronize()
        time.sleep(COLD_IDLE_S)
        c_first = warmup + 2 * steps
        _, c_step, (_, c_k3), c_mhz = timed_run(int2_step, c_first, 0, n_cold, marks_per_step=True)
        trace.update(cold_step_us=c_step, cold_history_us=c_k3, cold_history_mhz=c_mhz)
        c_launch, c_stp, _ = byte_totals(c_first, n_cold)
        c_k3_gbs = c_launch / (sum(c_k3) * 1e-6) / 1e9
        cold = {"idle_s": COLD_IDLE_S, "warmup": 0, "steps": n_cold,
                "us_per_step": round(sum(c_step) / n_cold, 2), "history_us": round(sum(c_k3) / n_cold, 2),
                "history_frac": round(c_k3_gbs / PEAK_HBM_GBS, 4),
                "quarters_step_us": quarters(c_step), "quarters_history_us": quarters(c_k3),
                "quarters_history_mhz": quarters(c_mhz), "min_history_mhz": round(min(c_mhz), 1),
                "what": "the same steps after 1 s of GPU idle, with no warm-up; history_mhz is the shader "
                        "clock over the history launch"}

    base = None
    if args.bf16_baseline == "on" or (args.bf16_baseline == "auto" and args.workload in ("b32-100k-g128",
                                                                                       "b32-100k-g64")):
        base = bf16_baseline(ok, W, HipEvent, torch, w, layout, lens_t, appends, q_all, kn_all, vn_all, max_len,
                             n_layers, stream, dims, hkv, hq, warmup, steps, args.history_target)
        if base is not None:
            base["int2_step_speedup"] = round(base["us_per_step"] / (step_ms * 1e3), 3)
            base["int2_history_speedup"] = round(base["history_us"] / k3_avg, 3)
            base["byte_ratio"] = round(base["bytes_per_step"] / (step_tot / steps), 3)

    cpu = None
    if workers is not None:
        hosted = {"r_k32": r_k.cpu().numpy(), "r_v32": r_v.cpu().numpy(),
                  "clip_k": c_k.cpu().numpy(), "clip_v": c_v.cpu().numpy()}
        try:
            cpu = cpu_baseline(workers, model, layout, hosted, lens_step[warmup + steps - 1])
        finally:
            workers.close()

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(step_ms, 4),
        "us_per_step": round(step_ms * 1e3, 2),
        # per-step latency from the next `steps` steps, with an event between
        # consecutive steps (the events cost a few µs per step)
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
                     "avg_us": round(k3_avg, 2),
                     "bytes_per_launch": int(launch_tot / len(k3_us)),
                     "launches_timed": {"every": every, "count": len(k3_us),
                                        "what": "history launches of the timed steps that ran between their "
                                                "own HIP start/stop events on the launch stream"},
                     "read_ceiling_gbs": probes["read_ceiling_gbs"],
                     "frac_of_read_ceiling": round(k3_gbs / probes["read_ceiling_gbs"], 4),
                     "unit_bytes": {"history_token_head": hist_unit_bytes(w.group_size),
                                    "bf16_token_head": 512}},
        "quarters": {"history_us": quarters(k3_us), "history_mhz": quarters(k3_mhz),
                     "min_history_mhz": round(min(k3_mhz), 1)},
        "step_vs_history": round((total_us / steps) / k3_avg, 4),
        "probes": probes,
        "cold_start": cold,
        "cpu_baseline": cpu,
        "bf16_baseline": base,
        "calibration_s": round(calib_s, 2),
    }
    if layout.chain_len:
        res["unique_value"] = round(unique_tot / (total_us * 1e-6) / 1e9, 2)
    if args.trace_file:
        with open(args.trace_file, "w") as f:
            json.dump(trace, f)
    print(json.dumps(res), flush=True)
    return 0


def bf16_baseline(ok, W, HipEvent, torch, w, layout, lens_t, appends, q_all, kn_all, vn_all, max_len,
                  n_layers, stream, dims, hkv, hq, warmup, steps, target):
    """The same steps on an all-bf16 cache (oscar_bf16_append +
    oscar_bf16_decode), after the same bandwidth settle as the INT2 steps."""
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
    n = min(warmup + steps, appends)
    steps = min(steps, n)
    warmup = n - steps
    ev_b = [HipEvent() for _ in range(steps)]
    ev_a = [HipEvent() for _ in range(steps)]
    m0, m1 = HipEvent(), HipEvent()

    def one(s: int, opts):
        ok.oscar_bf16_append(dims, structs[s], kn_all[s], vn_all[s], stream)
        ok.oscar_bf16_decode(dims, structs[s], q_all[s], max_len, wsb, nb, out, None, stream, options=opts)

    bandwidth_probes(ok, torch, HipEvent, stream, settle_s=0.2)
    plain = ok.make_options(history_target=target)
    for s in range(warmup):
        one(s, plain)
    torch.cuda.synchronize()
    opts = [ok.make_options(0, target, ev_b[i], ev_a[i]) for i in range(steps)]
    m0.record(stream)
    for i in range(steps):
        one(warmup + i, opts[i])
    m1.record(stream)
    m1.synchronize()
    total_us = 1e3 * m0.elapsed_ms(m1)
    hist_us = [1e3 * ev_b[i].elapsed_ms(ev_a[i]) for i in range(steps)]
    hist_b = [int(lens_t[warmup + i].sum()) * hkv * 512 for i in range(steps)]
    step_b = [hb + w.batch * hq * 128 * (2 + 4) + w.batch * hkv * 512 for hb in hist_b]
    del bcache, wsb
    torch.cuda.empty_cache()
    h_gbs = sum(hist_b) / (sum(hist_us) * 1e-6) / 1e9
    return {"us_per_step": round(total_us / steps, 2),
            "value": round(sum(step_b) / (total_us * 1e-6) / 1e9, 2), "unit": "GB/s",
            "history_us": round(sum(hist_us) / steps, 2), "history_gbs": round(h_gbs, 1),
            "history_frac": round(h_gbs / PEAK_HBM_GBS, 4), "bytes_per_step": int(sum(step_b) / steps),
            "fill_s": round(fill_s, 1),
            "what": "oscar_bf16_append + oscar_bf16_decode over the same tokens, all in bf16 pages"}


if __name__ == "__main__":
    sys.exit(main())
