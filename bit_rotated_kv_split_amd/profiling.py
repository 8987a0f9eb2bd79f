"""Summaries of rocprofv3 output for the decode path (profiling aid).

    python -m bit_rotated_kv_split_amd.profiling stats <run_kernel_stats.csv> [--match a,b,...]
    python -m bit_rotated_kv_split_amd.profiling traffic <fetch_counter_collection.csv>
        <write_counter_collection.csv> --kernel hist_mfma --workload b32-100k-g128
        --name mfma [--out profiles/traffic.json]
    python -m bit_rotated_kv_split_amd.profiling counters <counter_collection.csv> --kernel hist_mfma

`traffic` turns the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch)
of the history kernel into bytes per launch.  Each counter is scaled by
what it reads for the 2 GiB device copy that `bench.py --copy-probe` runs in
the same process (copy bytes / counter bytes), so a counter that covers
only part of the memory channels is corrected.  The record carries a hash of
the decode kernels' code (csrc/decode*, csrc/*.h, comments excluded);
`bench.py` reports it only while that hash matches the code it runs.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sys

COPY_BYTES = 2 << 30


def _kernel_rows(path: str):
    return list(csv.DictReader(open(path)))


def stats(path: str, match: list[str] | None = None) -> str:
    rows = _kernel_rows(path)
    out = ["| kernel | calls | average µs | min µs | max µs |", "|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if match and not any(m in name for m in match):
            continue
        out.append(f"| `{name[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    return "\n".join(out)


def _counter_values(path: str, counter: str):
    """{kernel name: [value per dispatch]} and the copy-probe reading."""
    per = collections.defaultdict(list)
    copy = []
    for r in _kernel_rows(path):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        name = r["Kernel_Name"]
        if "copyBuffer" in name:
            copy.append((int(r["Grid_Size"]), v))
        else:
            per[name].append(v)
    big = max(copy) if copy else None
    return per, (big[1] if big else None)


def counters(path: str, kernel: str) -> dict:
    res = collections.defaultdict(list)
    for r in _kernel_rows(path):
        if kernel in r["Kernel_Name"]:
            res[r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in res.items()}


def derived(vals: dict, page_heads: float, simds: int = 1024, xcds: int = 8) -> dict:
    """Per-page instruction counts and busy fractions from the SQ counters.
    A wave64 vector instruction occupies its SIMD for 4 cycles (16 lanes a
    cycle); GRBM_GUI_ACTIVE is summed over the XCDs, so the kernel's cycles
    are GRBM_GUI_ACTIVE / xcds; SQ_VALU_MFMA_BUSY_CYCLES is summed over the
    SIMDs."""
    out = {}
    cycles = vals.get("GRBM_GUI_ACTIVE", 0.0) / xcds
    if page_heads > 0:
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA"):
            if k in vals:
                out[f"{k} per page-head"] = vals[k] / page_heads
    if cycles > 0:
        if "SQ_INSTS_VALU" in vals:
            out["vector ALU busy (4 cycles per instruction)"] = vals["SQ_INSTS_VALU"] * 4 / simds / cycles
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            out["matrix core busy"] = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cycles
    return out


def _code_only(text: str) -> str:
    """C++ source without comments, blank lines or indentation, so
    that editing a comment does not retire the traffic records.  Text after
    // is dropped line by line (no string literal in the hashed files holds
    //)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = []
    for ln in text.splitlines():
        ln = re.sub(r"//.*$", "", ln).strip()
        if ln:
            lines.append(ln)
    return "\n".join(lines)


def source_sha(root: str) -> str:
    """Hash of the decode kernels' code (csrc/decode*, csrc/*.h), comments
    excluded."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(root, "bit_rotated_kv_split_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.startswith("decode") or name.endswith(".h"):
            h.update(_code_only(open(os.path.join(d, name), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def traffic(fetch_csv: str, write_csv: str, kernel: str) -> dict:
    res = {}
    for tag, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        per, copy_kib = _counter_values(path, counter)
        vals = [v for name, vs in per.items() if kernel in name for v in vs]
        if not vals or not copy_kib:
            raise SystemExit(f"no {counter} readings for {kernel} or for the copy probe in {path}")
        factor = COPY_BYTES / (copy_kib * 1024)
        res[tag] = {"kib_per_dispatch": sum(vals) / len(vals), "dispatches": len(vals),
                    "copy_probe_kib": copy_kib, "scale": factor,
                    "bytes": sum(vals) / len(vals) * 1024 * factor}
    res["bytes_per_launch"] = int(res["fetch"]["bytes"] + res["write"]["bytes"])
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--match", default="")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--kernel", required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--name", required=True)
    b.add_argument("--out", default="")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--kernel", required=True)
    c.add_argument("--page-heads", type=float, default=0.0,
                   help="64-token pages x KV heads one dispatch processes (adds per-page and busy figures)")
    c.add_argument("--simds", type=int, default=1024)
    c.add_argument("--xcds", type=int, default=8)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats(args.csv, [m for m in args.match.split(",") if m]))
    elif args.cmd == "counters":
        vals = counters(args.csv, args.kernel)
        for k, v in sorted(vals.items()):
            print(f"{k}: {v:.6g}")
        for k, v in derived(vals, args.page_heads, args.simds, args.xcds).items():
            print(f"{k}: {v:.4g}")
    else:
        rec = traffic(args.fetch_csv, args.write_csv, args.kernel)
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        rec["source_sha"] = source_sha(root)
        print(json.dumps(rec, indent=1))
        if args.out:
            data = json.load(open(args.out)) if os.path.exists(args.out) else {}
            data[f"{args.workload}/{args.name}"] = rec
            json.dump(data, open(args.out, "w"), indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
