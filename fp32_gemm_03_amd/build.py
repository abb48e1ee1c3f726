"""Build the gfx950 SGEMM library in-tree: ``fp32_gemm_03_amd/libsgemm_mi355x.so``.

``python -m fp32_gemm_03_amd.build`` compiles it; ``--asm DIR`` also writes the
device assembly (``.s``) for resource-usage checks (VGPR / AGPR counts, LDS
bytes, scratch); ``--resources`` prints every kernel's register, LDS and
scratch use read from the built library's gfx950 code object.
"""
from __future__ import annotations

import argparse
import os
import re
import shutil
import subprocess
import tempfile

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


def _llvm_tool(name: str) -> str:
    path = os.path.join("/opt/rocm/llvm/bin", name)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found (ROCm's LLVM tools are needed to read the code object)")
    return path


def kernel_resources(library: str = LIBRARY) -> dict:
    """``{kernel symbol: {field: int}}`` from the AMDGPU metadata of the
    library's gfx950 code object: ``vgpr_count``, ``agpr_count``,
    ``sgpr_count``, ``vgpr_spill_count``, ``sgpr_spill_count``,
    ``private_segment_fixed_size`` (scratch bytes per lane) and
    ``group_segment_fixed_size`` (LDS bytes).  The code object is the one this
    build wrote into the library's offload bundle."""
    fields = ("vgpr_count", "agpr_count", "sgpr_count", "vgpr_spill_count", "sgpr_spill_count",
              "private_segment_fixed_size", "group_segment_fixed_size")
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin")
        co = os.path.join(d, "gfx950.co")
        subprocess.run([_llvm_tool("llvm-objcopy"), "--dump-section=.hip_fatbin=" + fat, library,
                        os.path.join(d, "copy.so")], check=True, capture_output=True)
        subprocess.run([_llvm_tool("clang-offload-bundler"), "--type=o", "--unbundle",
                        "--targets=hipv4-amdgcn-amd-amdhsa--" + ARCH, "--input=" + fat,
                        "--output=" + co], check=True, capture_output=True)
        notes = subprocess.run([_llvm_tool("llvm-readelf"), "--notes", co], check=True,
                               capture_output=True, text=True).stdout
    out = {}
    # the kernel list is a YAML sequence under "amdhsa.kernels:"; its entries
    # start at "- ." with the least indentation of any such line (the
    # kernels' argument lists nest deeper) and hold ".name:" and the fields
    # above, one per line
    notes = notes[notes.find("amdhsa.kernels:"):]
    dashes = [len(m.group(1)) for m in re.finditer(r"^( *)- \.", notes, flags=re.M)]
    if not dashes:
        return out
    entry_re = r"^" + " " * min(dashes) + r"- (?=\.)"
    for entry in re.split(entry_re, notes, flags=re.M):
        m = re.search(r"^\s*\.name:\s+(\S+)", entry, flags=re.M)
        if not m or not m.group(1).startswith("_Z"):
            continue
        rec = {}
        for f in fields:
            fm = re.search(r"^\s*\." + f + r":\s+(\d+)", entry, flags=re.M)
            if fm:
                rec[f] = int(fm.group(1))
        out[m.group(1)] = rec
    return out


def demangle(names):
    """Readable kernel names (``c++filt``), in the order given; the mangled
    names where no demangler is installed."""
    names = list(names)
    tool = shutil.which("c++filt")
    if not names or tool is None:
        return names
    res = subprocess.run([tool], input="\n".join(names), check=True,
                         capture_output=True, text=True).stdout.splitlines()
    return res if len(res) == len(names) else names


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", metavar="DIR", help="also write device assembly here")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--resources", action="store_true",
                    help="print each kernel's registers, spills, scratch and LDS from the built library")
    args = ap.parse_args()
    if args.resources:
        res = kernel_resources()
        for name, pretty in zip(res, demangle(res)):
            r = res[name]
            print(f"{r.get('private_segment_fixed_size', -1):5d} B scratch  "
                  f"v{r.get('vgpr_count', -1):3d} a{r.get('agpr_count', -1):3d} "
                  f"spill {r.get('vgpr_spill_count', -1):3d}  lds {r.get('group_segment_fixed_size', -1):6d}  "
                  f"{pretty}")
        return
    print(build(verbose=args.verbose))
    if args.asm:
        for p in write_asm(args.asm):
            print(p)


if __name__ == "__main__":
    main()
