"""Summaries of rocprofv3 CSV output for the SGEMM kernels.

    python -m fp32_gemm_03_amd.rocprof_summary stats DIR [--last N] [--by-grid]
        per-kernel call count and durations from DIR/*_kernel_stats.csv; with
        --last, also each kernel's mean over its last N dispatches in
        DIR/*_kernel_trace.csv (the timed launches after a benchmark's warm-up);
        with --by-grid, each kernel's dispatches split by grid size (one
        kernel launched on several problem shapes)
    python -m fp32_gemm_03_amd.rocprof_summary counters DIR [DIR ...]
        per-kernel mean of every counter over its dispatches (*_counter_collection.csv)
    python -m fp32_gemm_03_amd.rocprof_summary traffic --fetch D --write D \\
            --copy-fetch D --copy-write D --copy-bytes N --kernel SUBSTR
        HBM bytes per launch of the kernel whose name contains SUBSTR: the
        FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch) each scaled by
        what the same counter reads for a plain copy kernel of N bytes

The counter CSV has one row per (dispatch, counter); counters are already
reduced over the device's hardware blocks by rocprofv3.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import statistics

COPY_KERNEL_SUBSTR = "copyBuffer"


def _one(dirpath, suffix):
    hits = sorted(glob.glob(os.path.join(dirpath, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {dirpath}")
    return hits[0]


def kernel_stats(dirpath):
    with open(_one(dirpath, "_kernel_stats.csv")) as f:
        rows = list(csv.DictReader(f))
    return [{"name": r["Name"], "calls": int(r["Calls"]), "total_ns": float(r["TotalDurationNs"]),
             "avg_ns": float(r["AverageNs"]), "min_ns": float(r["MinNs"]),
             "max_ns": float(r["MaxNs"]), "pct": float(r["Percentage"])} for r in rows]


def trace_durations(dirpath):
    """``{kernel_name: [duration_ns per dispatch, in dispatch order]}`` from the kernel trace."""
    with open(_one(dirpath, "_kernel_trace.csv")) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    out = collections.defaultdict(list)
    for r in rows:
        out[r["Kernel_Name"]].append(float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def trace_by_grid(dirpath):
    """``{(kernel_name, grid_x): [duration_ns per dispatch, in dispatch order]}``."""
    with open(_one(dirpath, "_kernel_trace.csv")) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    out = collections.defaultdict(list)
    for r in rows:
        out[(r["Kernel_Name"], int(r["Grid_Size_X"]))].append(
            float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def counters(dirpath):
    """``{kernel_name: {counter: [value per dispatch]}}`` plus durations under '_duration_ns'."""
    with open(_one(dirpath, "_counter_collection.csv")) as f:
        rows = list(csv.DictReader(f))
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    seen = set()
    for r in rows:
        k = r["Kernel_Name"]
        out[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        d = (k, r["Dispatch_Id"])
        if d not in seen:
            seen.add(d)
            out[k]["_duration_ns"].append(float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def _match(table, substr):
    names = [k for k in table if substr in k]
    if len(names) != 1:
        raise KeyError(f"{len(names)} kernels match {substr!r}: {names}")
    return names[0]


def traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes, kernel):
    cf = counters(copy_fetch_dir)
    cw = counters(copy_write_dir)
    cfk = _match(cf, COPY_KERNEL_SUBSTR)
    cwk = _match(cw, COPY_KERNEL_SUBSTR)
    fetch_scale = copy_bytes / (statistics.mean(cf[cfk]["FETCH_SIZE"]) * 1024.0)
    write_scale = copy_bytes / (statistics.mean(cw[cwk]["WRITE_SIZE"]) * 1024.0)
    f = counters(fetch_dir)
    w = counters(write_dir)
    fk = _match(f, kernel)
    wk = _match(w, kernel)
    fetch = statistics.mean(f[fk]["FETCH_SIZE"]) * 1024.0 * fetch_scale
    write = statistics.mean(w[wk]["WRITE_SIZE"]) * 1024.0 * write_scale
    return {"kernel": fk, "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
            "hbm_bytes_per_launch": fetch + write, "fetch_scale": fetch_scale,
            "write_scale": write_scale, "copy_bytes": copy_bytes,
            "dispatches": len(f[fk]["FETCH_SIZE"])}


def _print_stats(dirpath, last=0, by_grid=False):
    tr = trace_durations(dirpath) if last else {}
    grids = trace_by_grid(dirpath) if by_grid else {}
    for r in kernel_stats(dirpath):
        print(f"{r['name']}\n    calls {r['calls']}  avg {r['avg_ns'] / 1e6:.4f} ms  "
              f"min {r['min_ns'] / 1e6:.4f} ms  max {r['max_ns'] / 1e6:.4f} ms  "
              f"total {r['total_ns'] / 1e6:.3f} ms  ({r['pct']:.2f}%)")
        d = tr.get(r["name"], [])[-last:] if last else []
        if d:
            print(f"    last {len(d)} dispatches: avg {statistics.mean(d) / 1e6:.4f} ms")
        for (name, gx), ds in sorted(grids.items(), key=lambda kv: kv[0][1]):
            if name != r["name"]:
                continue
            tail = ds[-last:] if last else ds
            print(f"    grid {gx} threads: {len(ds)} dispatches, avg {statistics.mean(ds) / 1e6:.4f} ms"
                  + (f", last {len(tail)} avg {statistics.mean(tail) / 1e6:.4f} ms" if last else ""))


def _print_counters(dirpath):
    for k, cs in counters(dirpath).items():
        print(k)
        for c, vals in sorted(cs.items()):
            print(f"    {c:32s} mean {statistics.mean(vals):.6g}  (n={len(vals)})")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--last", type=int, default=0)
    s.add_argument("--by-grid", action="store_true")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    t = sub.add_parser("traffic")
    for name in ("fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument("--" + name, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", required=True)
    args = ap.parse_args()
    if args.cmd == "stats":
        _print_stats(args.dir, args.last, args.by_grid)
    elif args.cmd == "counters":
        for d in args.dirs:
            print(f"== {d}")
            _print_counters(d)
    else:
        print(json.dumps(traffic(args.fetch, args.write, args.copy_fetch, args.copy_write,
                                 args.copy_bytes, args.kernel), indent=1))


if __name__ == "__main__":
    main()
