"""Memory-capacity and job-throughput model: the INT2 cache against an
all-bf16 cache under a fixed HBM budget.

    python -m bit_rotated_kv_split_amd.capacity [--context 100000] [--jobs 32] [--budgets-gb 288,80]

The pages report that the smaller history lets a server hold more requests
in the same memory, which raises job-level throughput at large batch
(page "Together AI 开源 OSCAR…", section "结果": batch 32 at 100K; page
"超越TurboQuant…", the serving paragraph on a fixed memory budget).  Their
figure comes from a full serving stack; this module rebuilds the argument
from parts measured here:

- bytes per request: exact, from the cache layouts of this library (the
  INT2 cache: 64 + 256 bf16 tokens and 64-token INT2 history pages with
  their bf16 scale/zero; the all-bf16 cache: 64-token bf16 pages);
- concurrency: how many requests of the context fit in the budget after the
  model's bf16 weights and a reserve;
- attention time per layer and step: measured on the GPU with this
  library's decode step (oscar_decode_step; oscar_bf16_append +
  oscar_bf16_decode) at each batch size the model needs;
- the rest of the step: the bf16 weights read once per step at the
  measured device-copy bandwidth, a lower bound for the memory-bound
  projections and MLP of decode (no GEMM is run).

A job of J requests decodes in waves of at most the concurrency; its
throughput is J tokens per sum of the waves' step times.  Steady-state
throughput is the concurrency over the step time at that concurrency.
"""
from __future__ import annotations

import argparse
import json
import math
import sys
from dataclasses import dataclass

SINK, RECENT, PAGE, HEAD_DIM = 64, 256, 64, 128


@dataclass(frozen=True)
class ModelShape:
    name: str
    layers: int
    hidden: int
    q_heads: int
    kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    tied_embeddings: bool

    def layer_params(self) -> int:
        h, d = self.hidden, self.head_dim
        attn = h * self.q_heads * d * 2 + h * self.kv_heads * d * 2      # q, o; k, v
        return attn + 3 * h * self.intermediate                          # gate, up, down

    def weight_bytes(self) -> int:
        emb = self.vocab * self.hidden * (1 if self.tied_embeddings else 2)
        return 2 * (self.layers * self.layer_params() + emb)

    def weight_bytes_per_step(self) -> int:
        """bf16 bytes a decode step reads: every layer and the output head
        (the input embedding is a gather of a few rows)."""
        return 2 * (self.layers * self.layer_params() + self.vocab * self.hidden)


# Qwen3-8B: 36 layers, hidden 4096, 32 query / 8 KV heads of 128, MLP 12288,
# vocabulary 151936, separate input and output embeddings.
QWEN3_8B = ModelShape("Qwen3-8B", 36, 4096, 32, 8, 128, 12288, 151936, False)


def int2_block_bytes(group: int) -> int:
    """One 64-slot history page of one KV head: K and V codes, then a bf16
    scale/zero pair per group of each token's K and V."""
    return 4096 + 512 * (HEAD_DIM // group)


def request_kv_bytes(shape: ModelShape, context: int, mode: str, group: int = 128) -> int:
    """Cache bytes one request of `context` tokens holds over all layers."""
    per_head_token_bf16 = 2 * 2 * HEAD_DIM                 # K and V
    if mode == "bf16":
        per_head = math.ceil(context / PAGE) * PAGE * per_head_token_bf16
    elif mode == "int2":
        n_bf16 = min(context, SINK + RECENT)
        hist_pages = math.ceil(max(0, context - SINK - RECENT) / PAGE)
        per_head = (SINK + RECENT) * per_head_token_bf16 * (n_bf16 > 0) + hist_pages * int2_block_bytes(group)
    else:
        raise ValueError(mode)
    return shape.layers * shape.kv_heads * per_head


def bits_per_element(context: int, group: int = 128) -> float:
    """Stored bits per K or V element of one request (sink and recent bf16,
    history at 2 bits plus its per-group scale and zero)."""
    n_hist = max(0, context - SINK - RECENT)
    return (min(context, SINK + RECENT) * 16 + n_hist * (2 + 32 / group)) / context


def concurrency(shape: ModelShape, budget_bytes: float, reserve_bytes: float, context: int, mode: str,
                group: int = 128) -> int:
    free = budget_bytes - shape.weight_bytes() - reserve_bytes
    return max(0, int(free // request_kv_bytes(shape, context, mode, group)))


def wave_batches(jobs: int, cap: int) -> list[int]:
    if cap <= 0:
        return []
    full, rest = divmod(jobs, cap)
    return [cap] * full + ([rest] if rest else [])


def step_seconds(shape: ModelShape, attn_us_per_layer: float, copy_gbs: float) -> float:
    return shape.layers * attn_us_per_layer * 1e-6 + shape.weight_bytes_per_step() / (copy_gbs * 1e9)


def model_rows(shape: ModelShape, context: int, jobs: int, budgets_gb, reserve_gb: float, group: int,
               attn_us, copy_gbs: float):
    """attn_us(mode, batch) -> measured attention microseconds per layer and step."""
    rows = []
    for gb in budgets_gb:
        row = {"budget_gb": gb, "context": context, "jobs": jobs}
        for mode in ("int2", "bf16"):
            cap = concurrency(shape, gb * 1e9, reserve_gb * 1e9, context, mode, group)
            waves = wave_batches(jobs, cap)
            job_s = sum(step_seconds(shape, attn_us(mode, b), copy_gbs) for b in waves)
            steady_s = step_seconds(shape, attn_us(mode, cap), copy_gbs) if cap else float("inf")
            row[mode] = {"request_gb": round(request_kv_bytes(shape, context, mode, group) / 1e9, 3),
                         "concurrency": cap, "waves": waves,
                         "job_tokens_per_s": round(jobs / job_s, 1) if waves else 0.0,
                         "steady_tokens_per_s": round(cap / steady_s, 1) if cap else 0.0,
                         "step_ms_at_concurrency": round(steady_s * 1e3, 3) if cap else None}
        i, b = row["int2"], row["bf16"]
        row["job_throughput_ratio"] = round(i["job_tokens_per_s"] / b["job_tokens_per_s"], 2) \
            if b["job_tokens_per_s"] else None
        row["steady_throughput_ratio"] = round(i["steady_tokens_per_s"] / b["steady_tokens_per_s"], 2) \
            if b["steady_tokens_per_s"] else None
        row["concurrency_ratio"] = round(i["concurrency"] / b["concurrency"], 2) if b["concurrency"] else None
        rows.append(row)
    return rows


class AttentionTimer:
    """Times one layer's decode step on the GPU for a uniform batch of
    `context`-token requests: the INT2 cache (oscar_decode_step, demotion and
    append included) or the all-bf16 cache (oscar_bf16_append +
    oscar_bf16_decode).  Results are cached per (mode, batch)."""

    def __init__(self, shape: ModelShape, context: int, group: int, seed: int = 5, steps: int = 10,
                 warmup: int = 3):
        import torch
        from synth import configs
        from . import _lib as ok
        from . import workload as W
        from .hipevents import HipEvent
        from .kvcache import Rotation
        self.torch, self.ok, self.W, self.HipEvent, self.configs = torch, ok, W, HipEvent, configs
        self.shape, self.context, self.group, self.seed = shape, context, group, seed
        self.steps, self.warmup = steps, warmup
        self.cache = {}
        w = self._workload(1)
        model = W.SyntheticModel(w)
        qc, kc, vc = model.calibration()
        dims = ok.make_dims(shape.q_heads, shape.kv_heads, group)
        n = qc.shape[0]
        cws = torch.empty(ok.oscar_calibrate_workspace_bytes(dims, n), dtype=torch.uint8, device="cuda")
        hkv = shape.kv_heads
        rk = torch.empty((hkv, 128, 128), dtype=torch.float32, device="cuda")
        rv = torch.empty_like(rk)
        ck = torch.empty((hkv, 128), dtype=torch.float32, device="cuda")
        cv = torch.empty_like(ck)
        ok.oscar_calibrate(dims, n, torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(),
                           torch.from_numpy(vc).cuda(), w.clip_pct, rk, rv, ck, cv, None, None, cws, cws.numel())
        torch.cuda.synchronize()
        self.rot = Rotation(rk, rv, ck, cv)
        self.dims = dims

    def _workload(self, batch: int):
        s = self.shape
        return self.configs.Workload(f"capacity-b{batch}", self.seed, s.q_heads, s.kv_heads, self.group, batch,
                                     (self.context,) * batch, paged=True)

    def __call__(self, mode: str, batch: int) -> float:
        if batch <= 0:
            return 0.0
        key = (mode, batch)
        if key not in self.cache:
            self.cache[key] = self._measure(mode, batch)
        return self.cache[key]

    def _measure(self, mode: str, batch: int) -> float:
        import numpy as np
        torch, ok, W = self.torch, self.ok, self.W
        w = self._workload(batch)
        total = self.steps + self.warmup
        layout = W.Layout(w, None, extra_tokens=total)
        model = W.SyntheticModel(w)
        hq, hkv = self.shape.q_heads, self.shape.kv_heads
        stream = torch.cuda.current_stream().cuda_stream
        lens_t = layout.lens[None, :] + np.arange(1, total + 1)[:, None]
        seq_dev = torch.from_numpy(lens_t.astype(np.int32)).cuda()
        max_len = int(lens_t.max())
        q_all = torch.stack([W.queries_tensor(model, s, batch) for s in range(1, total + 1)])
        # appended tokens: the generator's values are immaterial to the time
        kn = torch.randn((total, batch, hkv, 128), device="cuda").to(torch.bfloat16)
        vn = torch.randn_like(kn)
        out = torch.empty((batch, hq, 128), dtype=torch.float32, device="cuda")
        if mode == "int2":
            from .kvcache import DecodeWorkspace
            cache = W.build_cache(w, layout, model, self.rot)
            ws = DecodeWorkspace(self.dims, batch, max_len)
            structs = [ok.make_cache(cache.pages, cache.n_pages, cache.sink_k, cache.sink_v, cache.recent_k,
                                     cache.recent_v, cache.page_table, cache.max_pages_per_req,
                                     seq_dev[t].data_ptr(), batch) for t in range(total)]

            def one(s):
                ok.oscar_decode_step(self.dims, self.rot.struct, structs[s], kn[s], vn[s], q_all[s], max_len,
                                     ws.buf, ws.nbytes, out, None, stream)
        else:
            cache = W.build_bf16_cache(w, layout, extra_tokens=total)
            structs = [ok.make_bf16_cache(cache.pages, cache.n_pages, cache.page_table, cache.max_pages_per_req,
                                          seq_dev[t].data_ptr(), batch) for t in range(total)]
            nb = ok.oscar_bf16_decode_workspace_bytes(self.dims, batch)
            wsb = torch.empty(nb, dtype=torch.uint8, device="cuda")

            def one(s):
                ok.oscar_bf16_append(self.dims, structs[s], kn[s], vn[s], stream)
                ok.oscar_bf16_decode(self.dims, structs[s], q_all[s], max_len, wsb, nb, out, None, stream)
        for s in range(self.warmup):
            one(s)
        torch.cuda.synchronize()
        e0, e1 = self.HipEvent(), self.HipEvent()
        e0.record(stream)
        for s in range(self.warmup, total):
            one(s)
        e1.record(stream)
        e1.synchronize()
        us = 1e3 * e0.elapsed_ms(e1) / self.steps
        del cache, structs
        torch.cuda.empty_cache()
        print(f"[capacity] {mode} batch {batch} x {self.context}: {us:.1f} us per layer step",
              file=sys.stderr, flush=True)
        return us


def copy_bandwidth_gbs() -> float:
    import torch
    from .hipevents import HipEvent
    nb = 2 << 30
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = HipEvent(), HipEvent()
    e0.record(stream)
    dst.copy_(src)
    e1.record(stream)
    e1.synchronize()
    gbs = 2 * nb / (e0.elapsed_ms(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--context", type=int, default=100_000)
    ap.add_argument("--jobs", type=int, default=32)
    ap.add_argument("--budgets-gb", default="288,80")
    ap.add_argument("--reserve-gb", type=float, default=8.0,
                    help="memory kept for activations, workspaces and the runtime")
    ap.add_argument("--group", type=int, default=128)
    ap.add_argument("--steps", type=int, default=10)
    args = ap.parse_args(argv)
    shape = QWEN3_8B
    budgets = [float(x) for x in args.budgets_gb.split(",")]
    copy_gbs = copy_bandwidth_gbs()
    timer = AttentionTimer(shape, args.context, args.group, steps=args.steps)
    rows = model_rows(shape, args.context, args.jobs, budgets, args.reserve_gb, args.group, timer, copy_gbs)
    for row in rows:
        row.update({"model": shape.name, "weights_gb": round(shape.weight_bytes() / 1e9, 3),
                    "weights_read_per_step_gb": round(shape.weight_bytes_per_step() / 1e9, 3),
                    "copy_gbs": round(copy_gbs, 1), "reserve_gb": args.reserve_gb, "group_size": args.group,
                    "bits_per_element": round(bits_per_element(args.context, args.group), 3),
                    "attn_us_per_layer": {f"{m}_b{b}": round(v, 1) for (m, b), v in sorted(timer.cache.items())}})
        print(json.dumps(row), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
