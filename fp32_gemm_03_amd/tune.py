"""Time every compiled kernel variant on a set of shapes and compare each
shape's fastest variant with the one the library's selection picks.

    python -m fp32_gemm_03_amd.tune [--shapes S1,S2,...] [--variants V1,V2,...] [--access M1,...]
    python -m fp32_gemm_03_amd.tune --plans MxNxK:V/S/W:V/S/W,...

A shape is a named synthetic workload (``square8192_normal`` ...) or MxNxK
(A, B ~ N(0,1), seed 3, alpha 1, beta 0; ``MxNxK_beta``: beta 1 with C ~
U[-1,1), so that the epilogue reads C).  Every launch goes through the C
ABI on one stream; the time per launch is HIP events around a run of
launches after about 30 ms of untimed ones (0.5 s after the GPU has idled,
so that the clock has ramped up).  Besides the forced variants,
two rows time the library's own choice: ``auto`` (``sgemm``) and ``auto+ws``
(``sgemm_ws`` with the workspace it asks for, which may split K or share the
K tiles of a last partial round of tiles over stream-K workers).  Where
``sgemm`` cuts C into pieces, a third row times its block as one launch.  The last block is a table of the selection
against the best variant per shape: the measurement the selection table in
``sgemm.hip`` was fitted to, repeatable on any MI355X.
"""
from __future__ import annotations

import argparse
import json
import sys
import time

DEFAULT_SHAPES = [
    "square256_u01", "ragged_1000x1023x999", "square1024_normal", "square2048_normal",
    "3072x3072x3072", "square4096_upm1", "5120x5120x5120", "6144x6144x6144", "7168x7168x7168",
    "square8192_normal", "10240x10240x10240", "square16384_normal", "lowk_16384x16384x128", "512x512x8192",
    "1024x1024x4096", "1024x8192x8192", "16384x1024x1024", "1024x16384x1024",
]


def _problem(shape):
    from . import inputs
    if shape in inputs.WORKLOADS:
        return inputs.workload_problem(shape)
    dims, _, opt = shape.lower().partition("_")
    M, N, K = (int(x) for x in dims.split("x"))
    if opt == "beta":  # C ~ U[-1, 1), beta = 1: the epilogue reads C
        return inputs.make_problem(M, N, K, dist="normal", seed=3, beta=1.0, c_fill="upm1", name=shape)
    if opt:
        raise ValueError(f"unknown shape option {opt!r} in {shape!r}")
    return inputs.make_problem(M, N, K, dist="normal", seed=3, name=shape)


_last_timed = None  # time.monotonic() at the end of the previous _time


def _time(launch, flops, stream, target_s=0.1, warmup_s=0.03):
    """Mean ms per launch and TFLOP/s over about target_s of launches, after
    about warmup_s of untimed ones (a fixed time rather than a count, so that
    the clock has settled whatever the launch length).  After the GPU has
    idled (the first timing of a process, or a pause of over 0.5 s while the
    next shape's inputs are made) the warm-up is at least 0.5 s: from idle the
    clock takes longer than 30 ms to ramp up, and the first variant timed on
    2048^3 ran 3-4% slow without it."""
    import torch
    global _last_timed
    if _last_timed is None or time.monotonic() - _last_timed > 0.5:
        warmup_s = max(warmup_s, 0.5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    launch()
    e1.record(stream)
    torch.cuda.synchronize()
    est_ms = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(int(min(2000, max(3, warmup_s * 1e3 / est_ms)))):
        launch()
    torch.cuda.synchronize()
    e0.record(stream)
    launch()
    e1.record(stream)
    torch.cuda.synchronize()
    est_ms = max(e0.elapsed_time(e1), 1e-3)
    steps = int(min(500, max(5, target_s * 1e3 / est_ms)))
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    _last_timed = time.monotonic()
    return ms, flops / (ms * 1e-3) / 1e12


ACCESS_MODES = {"auto": 0, "buf128": 1, "buf32": 2, "checked": 3, "buf128ab": 4}


def time_plans(items, out=sys.stdout):
    """Time explicit plans against each other: each item is
    ``MxNxK:PLAN:PLAN...`` with a PLAN ``variant/splits/workers`` run through
    sgemm_variant (whole tiles, no cut), sgemm_splitk or sgemm_streamk with a
    workspace.  Each plan is timed twice, alternating, and its better run kept;
    the ratio is the last plan's rate over the first's."""
    import math
    import torch
    import fp32_gemm_03_amd as g

    g.load_library()
    stream = torch.cuda.Stream()
    ratios = []
    for item in items:
        shape, *plans = item.split(":")
        p = _problem(shape)
        a, b, c = p.A.cuda(), p.B.cuda(), p.C.cuda()
        args = (p.M, p.N, p.K, p.alpha, a, p.lda, b, p.ldb, p.beta, c, p.ldc)
        flops = 2.0 * p.M * p.N * p.K
        launches = []
        for plan in plans:
            v, sp, w = (int(x) for x in plan.split("/"))
            if w > 0:
                need = g.sgemm_streamk_workspace_size(v, w)
            elif sp > 1:
                need = g.sgemm_splitk_workspace_size(v, sp, p.M, p.N)
            else:
                need = 0
            ws = torch.empty(max(need // 4, 1) + 64, dtype=torch.float32, device="cuda")
            if w > 0:
                launches.append(lambda v=v, w=w, ws=ws: g.sgemm_streamk(v, w, *args, workspace=ws, stream=stream))
            elif sp > 1:
                launches.append(lambda v=v, sp=sp, ws=ws: g.sgemm_splitk(v, sp, *args, workspace=ws, stream=stream))
            else:
                launches.append(lambda v=v: g.sgemm_variant(v, *args, stream=stream))
        best = [0.0] * len(plans)
        for _ in range(2):
            for i, fn in enumerate(launches):
                best[i] = max(best[i], _time(fn, flops, stream)[1])
        ratios.append(best[-1] / best[0])
        cols = "  ".join(f"{pl} {g.sgemm_variant_name(int(pl.split('/')[0]))} {tf:.1f}"
                         for pl, tf in zip(plans, best))
        print(f"{shape:20s} {cols}  ratio {best[-1] / best[0]:.3f}", file=out, flush=True)
        del a, b, c, p, launches
        torch.cuda.empty_cache()
    if ratios:
        geo = math.exp(sum(math.log(r) for r in ratios) / len(ratios))
        print(f"{len(ratios)} shapes: ratio geometric mean {geo:.3f}, min {min(ratios):.3f}, "
              f"max {max(ratios):.3f}", file=out, flush=True)
    return ratios


def tune(shapes, variants=None, out=sys.stdout, accesses=("auto",)):
    import torch
    import fp32_gemm_03_amd as g

    g.load_library()
    if variants is None:
        variants = list(range(g.sgemm_variant_count()))
    stream = torch.cuda.Stream()
    table = []
    for shape in shapes:
        p = _problem(shape)
        a, b, c = p.A.cuda(), p.B.cuda(), p.C.cuda()
        args = (p.M, p.N, p.K, p.alpha, a, p.lda, b, p.ldb, p.beta, c, p.ldc)
        flops = 2.0 * p.M * p.N * p.K
        # the library's plans for these very operands (their alignment matters)
        cus = g.sgemm_device_shape()[0]
        o16 = g.sgemm_operands_load16(a, p.lda, b, p.ldb, c, p.ldc)
        _, auto, _, _, cut_r, cut_c, cut_v = g.sgemm_plan_pieces_for(cus, p.M, p.N, p.K, False, o16)
        rows = {}
        for v in variants:
            for acc in accesses:
                mode = ACCESS_MODES[acc]
                if g.sgemm_variant_access(v, mode, *args, stream=stream, check=False) != 0:
                    continue  # a build these operands do not allow
                ms, tf = _time(lambda: g.sgemm_variant_access(v, mode, *args, stream=stream),
                               flops, stream)
                name = g.sgemm_variant_name(v)
                rows[name if acc == "auto" else f"{name}:{acc}"] = (ms, tf)
        ms, tf = _time(lambda: g.sgemm(*args, stream=stream), flops, stream)
        rows["auto"] = (ms, tf)
        ws_bytes = g.sgemm_workspace_size(p.M, p.N, p.K)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda")
        ms, tf = _time(lambda: g.sgemm_ws(*args, workspace=ws, workspace_bytes=ws_bytes,
                                          stream=stream), flops, stream)
        rows["auto+ws"] = (ms, tf)
        _, ws_variant, splits, workers, _ = g.sgemm_plan_for(cus, p.M, p.N, p.K, True, o16)
        for name, (ms, tf) in rows.items():
            print(f"{shape:24s} {name:34s} {tf:8.2f} TFLOP/s {ms:10.4f} ms", file=out, flush=True)
        one = None
        if cut_r > 0:  # the same block as one launch over all of C, timed beside the cut
            one = _time(lambda: g.sgemm_variant(auto, *args, stream=stream), flops, stream)
            print(f"{shape:24s} {'auto as one launch':34s} {one[1]:8.2f} TFLOP/s {one[0]:10.4f} ms",
                  file=out, flush=True)
        forced = {k: v for k, v in rows.items() if k not in ("auto", "auto+ws")}
        best = min(forced, key=lambda k: forced[k][0])
        selected = g.sgemm_variant_name(auto)
        if cut_r > 0:  # C cut into pieces, one launch each
            parts = [f"{cut_r} x {cut_c}: {g.sgemm_variant_name(cut_v)}"]
            if cut_c < p.N:
                right = g.sgemm_plan_for(cus, cut_r, p.N - cut_c, p.K, False, o16)[1]
                parts.append(f"right {cut_r} x {p.N - cut_c}: {g.sgemm_variant_name(right)}")
            if cut_r < p.M:
                below = g.sgemm_plan_for(cus, p.M - cut_r, p.N, p.K, False, o16)[1]
                parts.append(f"below {p.M - cut_r} x {p.N}: {g.sgemm_variant_name(below)}")
            selected = ", ".join(parts) + f" (one launch of {g.sgemm_variant_name(auto)}: {one[1]:.2f})"
        table.append({"shape": shape, "M": p.M, "N": p.N, "K": p.K,
                      "selected": selected, "selected_ws": g.sgemm_variant_name(ws_variant),
                      "splits": splits, "workers": workers,
                      "auto_ms": rows["auto"][0], "auto_ws_ms": rows["auto+ws"][0],
                      "best": best, "best_ms": forced[best][0],
                      "auto_ws_tflops": rows["auto+ws"][1], "auto_tflops": rows["auto"][1],
                      "one_launch_tflops": one[1] if one else None})
        del a, b, c, ws, p
        torch.cuda.empty_cache()
    print("\n| shape | selected (`sgemm`) | with workspace (`sgemm_ws`: splits, stream-K workers) | "
          "auto TFLOP/s | auto+ws TFLOP/s | best forced variant | best / auto+ws time |", file=out)
    print("|---|---|---|---|---|---|---|", file=out)
    for r in table:
        print(f"| {r['shape']} | {r['selected']} | {r['selected_ws']} ({r['splits']}, {r['workers']}) | "
              f"{r['auto_tflops']:.2f} | {r['auto_ws_tflops']:.2f} | "
              f"{r['best']} | {r['best_ms'] / r['auto_ws_ms']:.3f} |", file=out)
    print(json.dumps(table), file=out, flush=True)
    return table


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--shapes", default=",".join(DEFAULT_SHAPES))
    ap.add_argument("--variants", default=None, help="comma-separated variant indices (default: all)")
    ap.add_argument("--plans", default=None,
                    help="comma-separated MxNxK:v/s/w:v/s/w items: time those plans against each other")
    ap.add_argument("--access", default="auto",
                    help="comma-separated access modes to time each variant in: "
                         + ", ".join(ACCESS_MODES) + " (default: auto, the variant's own choice)")
    args = ap.parse_args()
    if args.plans:
        time_plans(args.plans.split(","))
        return
    variants = None if args.variants is None else [int(x) for x in args.variants.split(",")]
    accesses = args.access.split(",")
    for acc in accesses:
        if acc not in ACCESS_MODES:
            ap.error(f"unknown access mode {acc!r}")
    tune(args.shapes.split(","), variants, accesses=accesses)


if __name__ == "__main__":
    main()
