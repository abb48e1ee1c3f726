#!/usr/bin/env python3
"""FP32 SGEMM throughput on one MI355X.

One step is one C = alpha*A*B + beta*C call through the C ABI (the whole hot
path: tile loads, LDS staging, inner product, epilogue) on the square 8192^3
problem (A, B ~ N(0,1) float32, seed 3, alpha = 1, beta = 0, C zeroed), with
every operand already resident in HBM.  W untimed warm-up steps, then K timed
steps bracketed by device synchronisation; one JSON line on stdout.

  value      = 2*M*N*K*K_steps / (timed seconds) / 1e12      [TFLOP/s]
  roofline   = the kernel's average duration from HIP events recorded on the
               launch stream around every timed launch; achieved = 2MNK / that
               duration; peak = 157.3 TFLOP/s (FP32 matrix, 256 CU x 256 FLOP/clk
               x 2.4 GHz); traffic = HBM bytes per launch from rocprofv3
               FETCH_SIZE + WRITE_SIZE (scaled by a copy-kernel calibration), read
               from profiles/ when it was taken on the current kernel source,
               else null.
  secondary  = the same timing (after at least 50 ms of untimed launches, and
               with events only around the whole run of launches) for
               every other workload of the sweep: 4096^3, the low-K
               16384^2 x 128 problem (beta = 1), 256^3, the ragged
               1000 x 1023 x 999 problem (beta = -0.5), 1024^3, 2048^3 and
               16384^3, each with its fraction of the FP32 peak, of the HBM
               peak (algorithmic bytes: A, B, C read, C written) and of the
               larger of the two bounds.
  cpu_baseline = the float64 CPU oracle on a bounded band of rows of the same
               problem, on every host core (rank 0, N = 1 only).
  parity     = those oracle rows against the same rows of C after the first
               launch (from the workload's initial C), copied back before the
               warm-up: max error ratio and the 1e-5 pass rule.
               Every secondary entry carries its own cpu_baseline and parity:
               the oracle on the whole problem (its time, and every element
               of C after the first launch against it), or, at 16384^3, on a
               band of the first rows, labelled in its "sample".
  clocks     = the shader clock level sysfs reports for each GPU just before and
               after the timed run.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3  # 256 CU x 256 FLOP/clk x 2.4 GHz (FP32 MFMA)
# The VALU path is built without packed FP32 instructions; gfx950 still issues a
# wave-wide non-packed v_fma_f32 at the full FP32 vector rate (a probe loop of
# independent v_fma_f32 sustains ~124 TFLOP/s, above half of 157.3), so the VALU
# path is held to the same 157.3 TFLOP/s vector peak.
PEAK_VALU_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# The pass rule against the oracle: max |C - ref| / (|alpha| sum_k |A_ik B_kj| + |beta C_ij| + 1e-30)
TOLERANCE = 1e-5
# Elements of C (rows x N) copied back after the first launch for the parity check.
CAPTURE_ELEMENTS = 1 << 25
WORKLOAD = "square8192_normal"
# Reported beside the main line: the other square size the metric names, the
# low-K shape, whose bound is taken as the larger of its FLOP time at the FP32
# peak and its algorithmic bytes at the HBM peak, and the rest of the sweep.
SECONDARY = ("square4096_upm1", "lowk_16384x16384x128", "square256_u01", "ragged_1000x1023x999",
             "square1024_normal", "square2048_normal", "square16384_normal")
# Each secondary workload is checked against the oracle too: the whole
# problem, except where that takes minutes of host time (16384^3, about
# 3 minutes on 16 cores), where a band of the first rows is used, labelled so.
BAND_ONLY = ("square16384_normal",)
BAND_SECONDS = 6.0
BAND_CAPTURE_ROWS = 2048


def _code_tokens(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed, so that a
    comment edit does not count as a kernel change (string literals in these
    sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the code (not the comments) the kernels are built from: the
    kernel templates and the variant table that instantiates them.  Host
    logic (argument checks, the shape-to-variant choice, the launch) is left
    out, so changing it does not void a stored kernel measurement."""
    from fp32_gemm_03_amd import build as b
    h = hashlib.sha256()
    with open(os.path.join(b.CSRC, "sgemm_kernels.hpp"), encoding="utf-8") as f:
        h.update(_code_tokens(f.read()).encode())
    with open(os.path.join(b.CSRC, "sgemm.hip"), encoding="utf-8") as f:
        text = f.read()
    i, j = text.find("#define VALU_CFG"), text.find("constexpr int kNumVariants")
    h.update(_code_tokens(text[i:j] if 0 <= i < j else text).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, variant_name: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when there is none for this kernel or it predates the current source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload, {}).get(variant_name)
    if not entry or entry.get("source_hash") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def time_gpu(p, steps, warmup, path, variant=None, min_warmup_s=0.0, per_launch=True, capture_rows=0,
             info=None):
    """Launch on a dedicated stream; HIP events on that stream around every launch
    (with per_launch False only around the whole run, so that the host's event
    records do not leave a short kernel's queue empty).  After the `warmup`
    untimed launches, further untimed ones until about min_warmup_s has passed
    (so a short kernel after host work starts timing at a settled clock).
    With capture_rows > 0, the first `capture_rows` rows of C after the first
    launch (from the problem's initial C) are copied to the host and returned
    as a fourth value, for checking against the oracle.  With an `info` dict,
    info["variant"] is the variant the launches ran (the library's choice for
    these very operands, whose alignment it depends on, or the forced one)."""
    import torch
    import fp32_gemm_03_amd as g

    a = p.A.cuda()
    b = p.B.cuda()
    c = p.C.cuda()
    stream = torch.cuda.Stream()
    args = (p.M, p.N, p.K, p.alpha, a, p.lda, b, p.ldb, p.beta, c, p.ldc)
    if info is not None:
        info["variant"] = (g.sgemm_select_variant_for(path, p.M, p.N, p.K, a, p.lda, b, p.ldb, c, p.ldc)
                           if variant is None else variant)

    def step():
        if variant is None:
            g.sgemm_path(path, *args, stream=stream)
        else:
            g.sgemm_variant(variant, *args, stream=stream)

    torch.cuda.synchronize()
    first_rows = None
    if capture_rows > 0:
        step()
        torch.cuda.synchronize()
        first_rows = c[:capture_rows, :p.N].cpu().numpy().astype(np.float64)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if min_warmup_s > 0:
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < min_warmup_s:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_launch else 2)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        step()
        if per_launch:
            ev[i + 1].record(stream)
    if not per_launch:
        ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)] if per_launch else []
    total_ms = ev[0].elapsed_time(ev[-1])
    del a, b, c
    if capture_rows > 0:
        return total_ms, per_launch_ms, wall, first_rows
    return total_ms, per_launch_ms, wall


def cpu_baseline(p, target_s=10.0, gpu_rows=None, full=False):
    """The oracle timed on the whole problem (full) or on a band of rows
    0..r-1 sized to about target_s seconds; with gpu_rows (the GPU's first
    rows of C after its first launch), also the parity of those rows against
    the same oracle rows."""
    import oracle

    A, B = p.np("A"), p.np("B")
    Cin = p.np("C") if p.beta != 0 else None
    cores = oracle.nthreads()
    if full:
        rows2 = p.M
    else:
        rows = max(8, min(cores, p.M))
        t0 = time.perf_counter()
        oracle.sgemm_rows(p.M, p.N, p.K, p.alpha, A, p.lda, B, p.ldb, p.beta, Cin, p.ldc, 0, rows)
        t_probe = time.perf_counter() - t0
        rows2 = int(max(rows, min(p.M, rows * target_s / max(t_probe, 1e-3))))
        rows2 = min(p.M, max(rows, (rows2 // cores) * cores))
    t0 = time.perf_counter()
    ref, den = oracle.sgemm_rows(p.M, p.N, p.K, p.alpha, A, p.lda, B, p.ldb, p.beta, Cin, p.ldc, 0, rows2)
    t = time.perf_counter() - t0
    flops = 2.0 * rows2 * p.N * p.K
    sample = (f"the whole {p.M}x{p.N}x{p.K} problem ({rows2 * p.N} elements, float64 i-k-j loop), "
              f"{t:.1f} s" if rows2 == p.M else
              f"rows 0..{rows2 - 1} of the {p.M}x{p.N}x{p.K} problem "
              f"({rows2 * p.N} elements, float64 i-k-j loop), {t:.1f} s")
    out = {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
           "kind": "oracle", "sample": sample, "seconds": round(t, 3)}
    parity = None
    if gpu_rows is not None:
        r = min(rows2, gpu_rows.shape[0])
        err = oracle.max_error_ratio(gpu_rows[:r], ref[:r], den[:r])
        parity = {"rows": r, "elements": r * p.N, "max_err_ratio": err, "tolerance": TOLERANCE,
                  "pass": bool(err <= TOLERANCE),
                  "against": ("every element of the oracle's result" if r == p.M else
                              "the oracle's rows of the CPU baseline") +
                             "; C after the first launch from the workload's initial C"}
    del ref, den
    return out, parity


def gpu_clocks():
    """The current shader clock level of each GPU the driver lists, read from
    sysfs (pp_dpm_sclk, the line marked '*'); plain file reads, no program is
    started.  None where the files are not readable."""
    out = {}
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                cur = [line.strip() for line in f if line.rstrip().endswith("*")]
        except OSError:
            continue
        if cur:
            out[path.split("/")[4]] = cur[0].rstrip("* ").strip()
    return out or None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--path", choices=["auto", "valu", "mfma"], default="auto")
    ap.add_argument("--variant", type=int, default=None,
                    help="force one compiled kernel variant by index instead of the path's choice")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--shape", metavar="MxNxK",
                    help="time this square-workload recipe (N(0,1), seed 3) at another shape "
                         "instead of --workload (used for counter differencing)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", type=int, metavar="BYTES", default=0,
                    help="only run 5 plain device-to-device copies of BYTES bytes (the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this SGEMM runs on one GPU; multi-GPU runs are not part of it "
              "(C would split by row blocks of A, with B replicated and no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import fp32_gemm_03_amd as g
    from fp32_gemm_03_amd import inputs

    if not args.no_cpu_baseline:
        import oracle
        oracle.default()  # loaded (or compiled) before the GPU is initialised
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n, "copies": 5}), flush=True)
        return
    g.load_library()
    path = {"auto": g.SGEMM_PATH_AUTO, "valu": g.SGEMM_PATH_VALU, "mfma": g.SGEMM_PATH_MFMA}[args.path]

    if args.shape:
        M, N, K = (int(x) for x in args.shape.lower().split("x"))
        args.workload = f"square_recipe_{M}x{N}x{K}"
        w = inputs.Workload(args.workload, M, N, K, "normal", 3)
        p = inputs.make_problem(M, N, K, dist="normal", seed=3, name=args.workload)
    else:
        w = inputs.WORKLOADS[args.workload]
        p = inputs.workload_problem(args.workload)
    if args.variant is not None and g.sgemm_variant_name(args.variant) is None:
        print(f"bench.py: no variant {args.variant}", file=sys.stderr)
        sys.exit(2)
    print(f"bench: {args.workload}, {args.warmup} warm-up + {args.steps} timed", file=sys.stderr, flush=True)
    capture = 0 if args.no_cpu_baseline else max(1, min(p.M, CAPTURE_ELEMENTS // max(p.N, 1)))
    clocks_before = gpu_clocks()
    info = {}
    timed = time_gpu(p, args.steps, args.warmup, path, args.variant, capture_rows=capture, info=info)
    clocks_after = gpu_clocks()
    variant = info["variant"]
    vname = g.sgemm_variant_name(variant)
    print(f"bench: {args.workload} ran variant {vname}", file=sys.stderr, flush=True)
    total_ms, per_launch, wall = timed[:3]
    first_rows = timed[3] if capture else None
    ms_per_step = total_ms / args.steps
    value = w.flops / (ms_per_step / 1e3) / 1e12
    avg_kernel_ms = sum(per_launch) / len(per_launch)
    achieved = w.flops / (avg_kernel_ms / 1e3) / 1e12

    traffic = read_traffic(args.workload, vname)
    is_mfma = g.sgemm_variant_path(variant) == g.SGEMM_PATH_MFMA
    peak = PEAK_FP32_TFLOPS if is_mfma else PEAK_VALU_FP32_TFLOPS
    out = {
        "metric": "FP32 SGEMM TFLOP/s (2MNK/t)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": p.M, "N": p.N, "K": p.K,
                   "alpha": p.alpha, "beta": p.beta, "dist": w.dist, "seed": w.seed,
                   "variant": vname, "path": args.path},
        "pct_of_fp32_peak": round(100.0 * value / PEAK_FP32_TFLOPS, 2),
        "roofline": {"bound": "mfma" if is_mfma else "alu",
                     "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel_avg_ms": round(avg_kernel_ms, 4),
                     "kernel_median_ms": round(statistics.median(per_launch), 4),
                     "kernel_min_ms": round(min(per_launch), 4),
                     "algorithmic_flops_per_launch": w.flops,
                     "algorithmic_bytes_per_launch": w.algorithmic_bytes},
    }
    if not args.no_secondary and args.workload == WORKLOAD:
        out["secondary"] = []
        for name in SECONDARY:
            p2 = inputs.workload_problem(name)
            w2 = inputs.WORKLOADS[name]
            steps2 = max(args.steps, 100)
            full = name not in BAND_ONLY
            cap2 = 0 if args.no_cpu_baseline else (p2.M if full else BAND_CAPTURE_ROWS)
            print(f"bench: secondary {name}, {steps2} timed", file=sys.stderr, flush=True)
            info2 = {}
            timed2 = time_gpu(p2, steps2, args.warmup, path, args.variant, min_warmup_s=0.05, info=info2,
                              per_launch=False, capture_rows=cap2)
            t2 = timed2[0]
            v2 = info2["variant"]
            sec_s = t2 / steps2 / 1e3
            t_fp32 = w2.flops / (PEAK_FP32_TFLOPS * 1e12)
            t_hbm = w2.algorithmic_bytes / (PEAK_HBM_GBS * 1e9)
            entry = {
                "workload": name, "variant": g.sgemm_variant_name(v2),
                "value": round(w2.flops / sec_s / 1e12, 3), "unit": "TFLOP/s",
                "ms_per_step": round(sec_s * 1e3, 4), "steps": steps2,
                "pct_of_fp32_peak": round(100.0 * t_fp32 / sec_s, 2),
                "hbm_gbs": round(w2.algorithmic_bytes / sec_s / 1e9, 1),
                "pct_of_hbm_peak": round(100.0 * t_hbm / sec_s, 2),
                "roofline_bound": "mfma" if t_fp32 >= t_hbm else "hbm",
                "frac_of_roofline": round(max(t_fp32, t_hbm) / sec_s, 4)}
            if cap2:
                print(f"bench: oracle on {name} ({'whole problem' if full else 'row band'})",
                      file=sys.stderr, flush=True)
                entry["cpu_baseline"], entry["parity"] = cpu_baseline(
                    p2, target_s=BAND_SECONDS, gpu_rows=timed2[3], full=full)
            out["secondary"].append(entry)
            del p2, timed2
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["parity"] = cpu_baseline(p, gpu_rows=first_rows)
    out["clocks"] = {"before": clocks_before, "after": clocks_after,
                     "note": "idle snapshots around the timed run; the clock under load is "
                             "GRBM_GUI_ACTIVE over the kernel's duration (profiles/)"}
    cus, clk, peak_props = g.sgemm_device_fp32_peak(0)
    out["device"] = {"name": torch.cuda.get_device_name(0),
                     "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", ""),
                     "compute_units": cus, "peak_clock_mhz": clk / 1e3,
                     "fp32_peak_tflops_from_props": round(peak_props, 1)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
