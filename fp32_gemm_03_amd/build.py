"""Build the gfx950 SGEMM library in-tree: ``fp32_gemm_03_amd/libsgemm_mi355x.so``.

``python -m fp32_gemm_03_amd.build`` compiles it; ``--asm DIR`` also writes the
device assembly (``.s``) for resource-usage checks (VGPR / AGPR counts, LDS
bytes, scratch).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(CSRC, "sgemm.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, "sgemm_kernels.hpp"), os.path.join(INCLUDE, "sgemm.h")]
LIBRARY = os.path.join(PKG, "libsgemm_mi355x.so")
ARCH = "gfx950"

# Packed FP32 VALU instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False) -> str:
    """Compile the shared library (always recompiles) and return its path."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + COMMON + ["-shared", "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def write_asm(outdir: str) -> list:
    """Write the gfx950 device assembly of every source into ``outdir``."""
    os.makedirs(outdir, exist_ok=True)
    outs = []
    for src in SOURCES:
        out = os.path.join(outdir, os.path.basename(src).replace(".hip", f"-{ARCH}.s"))
        cmd = [hipcc()] + COMMON + ["--cuda-device-only", "-S", "-o", out, src]
        subprocess.run(cmd, check=True)
        outs.append(out)
    return outs


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", metavar="DIR", help="also write device assembly here")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(verbose=args.verbose))
    if args.asm:
        for p in write_asm(args.asm):
            print(p)


if __name__ == "__main__":
    main()
