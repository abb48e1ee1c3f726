"""Hardware counters equal the kernels' design counts (rocprofv3 --pmc).

Each case runs ``bench.py`` on a 2048^3 problem (A, B ~ N(0,1), alpha 1,
beta 0) with one variant forced, under ``rocprofv3 --pmc`` with a few SQ
counters, and checks every dispatch of the kernel:

* MFMA kernels: ``SQ_INSTS_MFMA`` is one v_mfma_f32_32x32x2_f32 per 32x32x2
  block of the (tile-padded) product, ``SQ_INSTS_VALU_MFMA_MOPS_F32`` x 512 is
  2 M'N'K', and no bf16/f16 matrix operation runs (true FP32 only);
* every kernel: ``SQ_LDS_BANK_CONFLICT`` is 0 and ``SQ_INSTS_LDS`` equals the
  per-wave LDS instruction count of the staging design times waves x K tiles;
* VALU kernels: ``SQ_INSTS_VALU_FMA_F32`` is M N K / 64 (one wave-wide FMA per
  64 multiply-adds, nothing packed, nothing else).
"""
import os
import shutil
import statistics
import subprocess
import sys
import tempfile

import pytest

import fp32_gemm_03_amd as g
from fp32_gemm_03_amd import rocprof_summary as rs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
S = 2048  # M = N = K


def _rocprof():
    exe = shutil.which("rocprofv3")
    if exe is None:
        pytest.skip("rocprofv3 not on PATH")
    return exe


def run_pmc(counters, variant):
    """Mean of each counter per dispatch of the forced variant's kernel."""
    exe = _rocprof()
    out = tempfile.mkdtemp(prefix="sgemm_pmc_", dir="/tmp")
    cmd = ["timeout", "-s", "KILL", "120", exe, "--pmc", *counters, "-d", out, "-o", "c",
           "--output-format", "csv", "--", sys.executable, os.path.join(ROOT, "bench.py"),
           "--no-cpu-baseline", "--no-secondary", "--shape", f"{S}x{S}x{S}",
           "--variant", str(variant), "--steps", "2", "--warmup", "1"]
    print("counters:", " ".join(counters), "variant", variant, flush=True)
    env = dict(os.environ, TMPDIR="/tmp")
    r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    try:
        table = rs.counters(out)
    except FileNotFoundError:
        pytest.fail(f"rocprofv3 wrote no counter file (exit {r.returncode}):\n{r.stdout[-3000:]}")
    kernels = [k for k in table if "sgemm_" in k]
    assert len(kernels) == 1, kernels
    k = kernels[0]
    vals = {c: table[k][c] for c in table[k] if not c.startswith("_")}
    shutil.rmtree(out, ignore_errors=True)
    for c in counters:
        if c not in vals:
            return None, k
        assert len(set(vals[c])) == 1, (c, vals[c])  # identical on every dispatch
    return {c: statistics.mean(v) for c, v in vals.items()}, k


def geometry(variant):
    _, bm, bn = g.sgemm_variant_tile(variant)
    name = g.sgemm_variant_name(variant)
    bk = int(name.split("_")[1].split("x")[2])
    return name, bm, bn, bk


def mfma_lds_per_wave(name, bm, bn, bk, threads, kt, mi):
    """LDS instructions of one wave over a tile's K loop of kt K tiles, and
    how many of them the compiler may fuse in pairs (ds_read2).

    A transposed (``_il`` and the plain loop): one A and one B fragment
    vector per k-step (BK / 2 steps per K tile), any two of which may fuse;
    writes: A as float4 per 4 rows, B as float4 along N, once per K tile,
    plus, on the interleaved schedule, the tile past the end that the last
    iteration stores unconditionally.
    A in K order, loaded straight into LDS (``_kcd``): per K tile one
    128-bit A read per block row and 4 k-steps (MI BK / 8) and one B read per
    k-step (BK / 2, which may fuse in pairs); no LDS store instruction (the
    buffer loads write LDS themselves)."""
    if "_kcd" in name:
        # with KG wave groups (``_kgN``) each wave covers bk / KG of every K
        # tile, then writes its 32 x 32 blocks to LDS once (four 128-bit
        # writes per block) and reads, per 4-float piece of the tile it
        # stores, that piece of every group (one 128-bit read each)
        kg = int(name.split("_kg")[1].split("_")[0]) if "_kg" in name else 1
        kx = bk // kg
        reads = mi * kx // 8 + kx // 2
        per, pairs = kt * reads, kt * (kx // 4)
        if kg > 1:
            blocks = (bm * bn // (32 * 32)) // (threads // 64 // kg)  # 32 x 32 blocks per wave
            per += 4 * blocks + kg * (bm * bn // 4) // threads
        return per, pairs
    reads = 2 * (bk // 2)
    writes = bm * bk // (4 * threads) + bk * bn // (4 * threads)
    stored = kt + 1 if "_il" in name else kt
    return kt * reads + stored * writes, kt * (bk // 2)


# the blocks the selection picks (every K-ordered block)
MFMA_CASES = [v for v in range(g.sgemm_variant_count()) if "_kcd" in (g.sgemm_variant_name(v) or "")]
VALU_CASES = [v for v in range(g.sgemm_variant_count()) if g.sgemm_variant_path(v) == g.SGEMM_PATH_VALU]
# MFMA kernels whose every LDS access is its own instruction (none of the
# chosen ones).  In the others the compiler fuses some pairs of fragment reads
# into one ds_read2 / ds_read2st64 instruction, so the counter lies between
# the fully fused and the unfused design count.
EXACT_LDS = set()


@pytest.mark.parametrize("variant", MFMA_CASES)
def test_mfma_counters_equal_design(variant):
    name, bm, bn, bk = geometry(variant)
    assert g.sgemm_variant_path(variant) == g.SGEMM_PATH_MFMA
    c, kernel = run_pmc(["SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_INSTS_MFMA",
                         "SQ_INSTS_VALU_MFMA_MOPS_F32"], variant)
    wm, wn = (int(x) for x in name.split("_w")[1].split("_")[0].split("x"))
    kg = int(name.split("_kg")[1].split("_")[0]) if "_kg" in name else 1
    waves_per_wg = kg * (bm // wm) * (bn // wn)
    threads = 64 * waves_per_wg
    tiles = (S // bm) * (S // bn)
    kt = S // bk
    # M', N', K' = the tile-padded sizes (here S is a multiple of every tile)
    assert c["SQ_INSTS_MFMA"] == S * S * S // (32 * 32 * 2)
    assert c["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512 == 2 * S ** 3
    assert c["SQ_LDS_BANK_CONFLICT"] == 0
    per, pairs = mfma_lds_per_wave(name, bm, bn, bk, threads, kt, wm // 32)
    design = tiles * waves_per_wg * per
    if variant in EXACT_LDS:
        assert c["SQ_INSTS_LDS"] == design, (kernel, per)
    else:
        fused = tiles * waves_per_wg * (per - pairs)  # every read pair fused
        assert fused <= c["SQ_INSTS_LDS"] <= design, (kernel, c["SQ_INSTS_LDS"], fused, design)


def test_mfma_runs_no_reduced_precision_matrix_ops():
    v = [i for i in MFMA_CASES if g.sgemm_variant_name(i) == "mfma_256x256x32_w128x64_kcd"][0]
    c, kernel = run_pmc(["SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                         "SQ_INSTS_VALU_MFMA_MOPS_F16"], v)
    if c is None:
        pytest.skip("bf16/f16 MFMA op counters not offered by this rocprofv3")
    assert c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] == 0
    assert c["SQ_INSTS_VALU_MFMA_MOPS_F16"] == 0
    assert c["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512 == 2 * S ** 3


@pytest.mark.parametrize("variant", VALU_CASES)
def test_valu_counters_equal_design(variant):
    name, bm, bn, bk = geometry(variant)
    assert g.sgemm_variant_path(variant) == g.SGEMM_PATH_VALU
    c, kernel = run_pmc(["SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_INSTS_VALU_FMA_F32",
                         "SQ_INSTS_MFMA"], variant)
    tm, tn = (int(x) for x in name.split("_t")[1].split("_")[0].split("x"))
    waves_per_wg = (bm // (8 * tm)) * (bn // (8 * tn))
    threads = 64 * waves_per_wg
    tiles = (S // bm) * (S // bn)
    kt = S // bk
    assert c["SQ_INSTS_VALU_FMA_F32"] == S ** 3 // 64
    assert c["SQ_INSTS_MFMA"] == 0
    assert c["SQ_LDS_BANK_CONFLICT"] == 0
    # per k: TM/4 + TN/4 float4 reads; per K tile: A and B float4 stores
    per = bk * (tm // 4 + tn // 4) + bm * bk // (4 * threads) + bk * bn // (4 * threads)
    assert c["SQ_INSTS_LDS"] == tiles * waves_per_wg * kt * per, (kernel, per)
