"""Per-workgroup phase times of the SGEMM kernels, from a measurement build.

    python -m fp32_gemm_03_amd.phases build
        compile csrc/sgemm.hip with SGEMM_PHASES into
        fp32_gemm_03_amd/libsgemm_phases.so (the library's own kernels, each
        with the phase stamps of sgemm_kernels.hpp switched on)
    python -m fp32_gemm_03_amd.phases run WORKLOAD:VARIANT [...]
        for each case (a named workload or MxNxK with the N(0,1) seed-3
        recipe; VARIANT an index or ``auto`` for the library's choice): 50
        untimed launches, then one launch whose log is read back, and one line
        of JSON with, over the workgroups of that launch:
          span_us          first entry to last end (real-time clock)
          start_spread_us  first to last workgroup entry
          clock_ghz        shader cycles / real time per workgroup (median)
          prologue, loop, epilogue
                           shader cycles per workgroup (median, max): entry to
                           the first K tile landed, the K loop, the epilogue
                           until its stores completed
          tile_body, tile_wait
                           the K loop split (medians of the per-workgroup
                           sums): the tiles' MFMAs and next-tile loads, and the
                           waits and barriers that end each tile
          mfma_cycles      the MFMA work of one wave over the K loop
                           (v_mfma_f32_32x32x2_f32: 64 cycles each)

The stamps are taken by lane 0 of each workgroup's first wave (its K loop and
epilogue stand for the workgroup's); they cost a few scalar instructions per K
tile, so this build is for splitting time between phases, not for the rates
of bench.py.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import subprocess
import sys

from . import build as _build

LIBRARY = os.path.join(_build.PKG, "libsgemm_phases.so")
SLOTS = 8


def build() -> str:
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [_build.hipcc()] + _build.COMMON + ["-DSGEMM_PHASES", "-shared", "-o", tmp] + _build.SOURCES
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def _load():
    if not os.path.exists(LIBRARY):
        raise FileNotFoundError(f"{LIBRARY} is missing: run `python -m fp32_gemm_03_amd.phases build`")
    lib = ctypes.CDLL(LIBRARY)
    i, f, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.sgemm_variant.argtypes = [i, i, i, i, f, vp, i, vp, i, f, vp, i, vp]
    lib.sgemm_variant.restype = i
    lib.sgemm_variant_name.argtypes = [i]
    lib.sgemm_variant_name.restype = ctypes.c_char_p
    lib.sgemm_variant_tile.argtypes = [i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.sgemm_variant_tile.restype = i
    lib.sgemm_select_variant_for.argtypes = [i, i, i, i, vp, i, vp, i, vp, i]
    lib.sgemm_select_variant_for.restype = i
    lib.sgemm_phase_read.argtypes = [vp, i]
    lib.sgemm_phase_read.restype = i
    return lib


def _problem(name):
    from . import inputs
    if name in inputs.WORKLOADS:
        return inputs.workload_problem(name)
    M, N, K = (int(x) for x in name.lower().split("x"))
    return inputs.make_problem(M, N, K, dist="normal", seed=3, name=name)


def run_case(lib, name, variant):
    import numpy as np
    import torch

    p = _problem(name)
    a, b, c = p.A.cuda(), p.B.cuda(), p.C.cuda()
    v = (lib.sgemm_select_variant_for(0, p.M, p.N, p.K, a.data_ptr(), p.lda, b.data_ptr(), p.ldb,
                                      c.data_ptr(), p.ldc) if variant == "auto" else int(variant))
    raw = lib.sgemm_variant_name(v)
    if raw is None:
        raise ValueError(f"no variant {variant}")
    vname = raw.decode()
    bm, bn = ctypes.c_int(), ctypes.c_int()
    lib.sgemm_variant_tile(v, ctypes.byref(bm), ctypes.byref(bn))
    wgs = math.ceil(p.M / bm.value) * math.ceil(p.N / bn.value)

    def launch():
        rc = lib.sgemm_variant(v, p.M, p.N, p.K, p.alpha, a.data_ptr(), p.lda, b.data_ptr(), p.ldb,
                               p.beta, c.data_ptr(), p.ldc, None)
        if rc != 0:
            raise RuntimeError(f"sgemm_variant returned {rc}")

    for _ in range(50):
        launch()
    torch.cuda.synchronize()
    launch()
    torch.cuda.synchronize()
    n = min(wgs, 65536)
    log = np.zeros(n * SLOTS, dtype=np.uint64)
    rc = lib.sgemm_phase_read(log.ctypes.data, n * SLOTS)
    if rc != 0:
        raise RuntimeError(f"sgemm_phase_read returned {rc}")
    r = log.reshape(n, SLOTS).astype(np.int64)
    cyc = np.diff(r[:, :4], axis=1)
    real_ns = (r[:, 7] - r[:, 6]) * 10.0
    k_tiles = math.ceil(p.K / int(vname.split("_")[1].split("x")[2]))
    wm, wn = (int(x) for x in vname.split("_w")[1].split("_")[0].split("x"))
    kg = int(vname.split("_kg")[1].split("_")[0]) if "_kg" in vname else 1
    mfma = (wm // 32) * (wn // 32) * (k_tiles * int(vname.split("_")[1].split("x")[2]) // kg // 2) * 64
    med = lambda x: int(np.median(x))
    out = {"workload": name, "variant": vname, "workgroups": int(wgs), "sampled": int(n),
           "span_us": round(float((r[:, 7].max() - r[:, 6].min()) * 10e-3), 2),
           "start_spread_us": round(float((r[:, 6].max() - r[:, 6].min()) * 10e-3), 2),
           "clock_ghz": round(float(np.median((r[:, 3] - r[:, 0]) / real_ns)), 3),
           "prologue": [med(cyc[:, 0]), int(cyc[:, 0].max())],
           "loop": [med(cyc[:, 1]), int(cyc[:, 1].max())],
           "epilogue": [med(cyc[:, 2]), int(cyc[:, 2].max())],
           "tile_body": med(r[:, 4]), "tile_wait": med(r[:, 5]), "k_tiles": k_tiles,
           "mfma_cycles": int(mfma) if vname.startswith("mfma") else None}
    del a, b, c
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("build")
    r = sub.add_parser("run")
    r.add_argument("cases", nargs="+", metavar="WORKLOAD:VARIANT")
    args = ap.parse_args()
    if args.cmd == "build":
        print(build())
        return
    lib = _load()
    for case in args.cases:
        name, _, variant = case.partition(":")
        print(json.dumps(run_case(lib, name, variant or "auto")), flush=True)


if __name__ == "__main__":
    sys.exit(main())
