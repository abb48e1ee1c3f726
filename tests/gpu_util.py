"""Helpers for the GPU parity tests: run the HIP library through its C ABI on
seeded inputs and compare with the float64 oracle under the pass rule
max |C_gpu - ref| / (|alpha| sum_k |A_ik||B_kj| + |beta||C_ij| + 1e-30) <= 1e-5."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fp32_gemm_03_amd as g
import oracle

TOL = 1e-5


def say(*args):
    """Name the case before a GPU step, flushed, so a hard failure still leaves it."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


GUARD = 256  # floats of NaN on each side of every operand buffer


def to_gpu(t: torch.Tensor, offset_floats: int = 0) -> tuple:
    """Copy a CPU tensor to the GPU inside a NaN-filled guard band; with
    ``offset_floats`` the data starts that many floats later (a deliberately
    misaligned base).  Returns ``(owner, first_index, base_address)``."""
    flat = t.contiguous().reshape(-1)
    first = GUARD + offset_floats
    owner = torch.full((first + flat.numel() + GUARD,), float("nan"), dtype=torch.float32,
                       device="cuda")
    owner[first:first + flat.numel()].copy_(flat)
    return owner, first, owner.data_ptr() + 4 * first


def run(p, variant=None, path=None, offsets=(0, 0, 0), stream=None, access=None):
    """Launch one SGEMM on ``p`` (an ``inputs.Problem``); returns the whole C buffer
    (M x ldc, float32, numpy) after the call, and checks that nothing outside the
    operands' extents was written."""
    oa, _, a = to_gpu(p.A, offsets[0])
    ob, _, b = to_gpu(p.B, offsets[1])
    oc, first, c = to_gpu(p.C, offsets[2])
    args = (p.M, p.N, p.K, p.alpha, a, p.lda, b, p.ldb, p.beta, c, p.ldc)
    if access is not None:
        g.sgemm_variant_access(variant, access, *args, stream=stream)
    elif variant is not None:
        g.sgemm_variant(variant, *args, stream=stream)
    elif path is not None:
        g.sgemm_path(path, *args, stream=stream)
    else:
        g.sgemm(*args, stream=stream)
    torch.cuda.synchronize()
    n = p.C.numel()
    host = oc.cpu().numpy()
    guard = np.concatenate([host[:first], host[first + n:]])
    assert np.all(np.isnan(guard)), "write outside C's extent"
    for o in (oa, ob):
        h = o.cpu().numpy()
        assert np.isnan(h[:GUARD]).all() and np.isnan(h[-GUARD:]).all(), "write into A or B"
    return host[first:first + n].reshape(p.C.shape)


def oracle_full(p):
    return oracle.sgemm(p.M, p.N, p.K, p.alpha, p.np("A"), p.lda, p.np("B"), p.ldb,
                        p.beta, p.np("C"), p.ldc)


def ratio_full(p, out, ref_den=None):
    ref, den = oracle_full(p) if ref_den is None else ref_den
    return oracle.max_error_ratio(out[:, :p.N], ref, den)


def ratio_points(p, out, rows, cols):
    ref, den = oracle.sgemm_points(p.M, p.N, p.K, p.alpha, p.np("A"), p.lda, p.np("B"),
                                   p.ldb, p.beta, p.np("C"), p.ldc, rows, cols)
    return oracle.max_error_ratio(out[rows, cols], ref, den)


def line_sample(M, N, n_lines=62, n_random=4096, seed=0):
    """The full-size sample: whole rows {0, M-1, n_lines seeded}, whole
    columns {0, N-1, n_lines seeded}, and n_random seeded points."""
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, n_lines)])).astype(np.int64)
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, n_lines)])).astype(np.int64)
    pr = rng.integers(0, M, n_random).astype(np.int32)
    pc = rng.integers(0, N, n_random).astype(np.int32)
    return rows, cols, pr, pc


def ratio_lines(p, out, n_lines=62, n_random=4096, seed=0):
    """Max error ratio over whole sampled rows and columns of C plus random
    points.  Row i of the sample is the oracle on A's row i alone (the rows
    gathered into a small problem); column j likewise on B's column j: the
    same products summed in the same order as over the full problem.
    Returns (ratio, rows, cols)."""
    M, N, K = p.M, p.N, p.K
    rows, cols, pr, pc = line_sample(M, N, n_lines, n_random, seed)
    A = p.A.numpy()[:, :K] if p.A.numel() else np.zeros((M, max(K, 1)), np.float32)
    B = p.B.numpy()[:, :N] if p.B.numel() else np.zeros((max(K, 1), N), np.float32)
    C = p.C.numpy()[:, :N] if p.beta != 0 else None
    As = np.ascontiguousarray(A[rows]).reshape(-1)
    Cr = np.ascontiguousarray(C[rows]).reshape(-1) if C is not None else None
    ref, den = oracle.sgemm(len(rows), N, K, p.alpha, As, K, np.ascontiguousarray(B).reshape(-1) if
                            p.ldb != N else p.np("B"), N, p.beta, Cr, N)
    r_rows = oracle.max_error_ratio(out[rows, :N], ref, den)
    Bs = np.ascontiguousarray(B[:, cols]).reshape(-1)
    Cc = np.ascontiguousarray(C[:, cols]).reshape(-1) if C is not None else None
    ref, den = oracle.sgemm(M, len(cols), K, p.alpha, p.np("A") if p.lda == K else
                            np.ascontiguousarray(A).reshape(-1), K, Bs, len(cols), p.beta, Cc, len(cols))
    r_cols = oracle.max_error_ratio(out[:, cols], ref, den)
    r_pts = ratio_points(p, out, pr, pc)
    return max(r_rows, r_cols, r_pts), rows, cols


def pad_untouched(p, out):
    """Columns N..ldc-1 of C are outside the matrix and must keep their sentinel bits."""
    if p.ldc == p.N:
        return True
    before = p.C.numpy()[:, p.N:]
    after = out[:, p.N:]
    return np.array_equal(before.view(np.uint32), after.view(np.uint32))


ACCESS_NAMES = {0: "auto", 1: "buf128", 2: "buf32", 3: "checked", 4: "buf128ab"}


def sum_family(variant, access):
    """Which kernel a build of a variant runs, as far as the order of its sums
    goes: the K-ordered direct-load kernel ("kc": the 128-bit and
    BUFFER_128_AB builds of the ``_kcd`` variants, every build of the 32 x 32
    and 32 x 64 blocks) or the register-staged one ("rs": the other
    ``_kcd`` builds, and every build of the other variants)."""
    name = g.sgemm_variant_name(variant)
    kc_access = (g.SGEMM_ACCESS_BUFFER_128, g.SGEMM_ACCESS_BUFFER_128_AB)
    if name.startswith("mfma_32x"):  # the small blocks: every build is the K-ordered kernel
        return "kc"
    return "kc" if name.endswith("_kcd") and access in kc_access else "rs"


def same_sum_order(variant, a1, a2):
    return sum_family(variant, a1) == sum_family(variant, a2)


def auto_access(p, variant, offsets=(0, 0, 0)):
    """The build SGEMM_ACCESS_AUTO runs for these arguments: the 128-bit
    one, else the one loading A and B 16 bytes at a time at 4-byte
    alignment, else the 32-bit one."""
    modes = allowed_accesses(p, offsets, variant)
    for m in (g.SGEMM_ACCESS_BUFFER_128, g.SGEMM_ACCESS_BUFFER_128_AB):
        if m in modes:
            return m
    return g.SGEMM_ACCESS_BUFFER_32


def allowed_accesses(p, offsets=(0, 0, 0), variant=None):
    """The access modes whose preconditions these arguments meet for a
    variant (the test operands are small, so the 31-bit offset bound always
    holds)."""
    modes = [g.SGEMM_ACCESS_BUFFER_32, g.SGEMM_ACCESS_CHECKED]
    aligned = offsets[1] % 4 == 0 and offsets[2] % 4 == 0
    ok128 = p.N % 4 == 0 and p.ldb % 4 == 0 and p.ldc % 4 == 0 and aligned
    if variant is not None and g.sgemm_variant_reads_a128(variant) == 1:
        ok128 = ok128 and p.K % 4 == 0 and p.lda % 4 == 0 and offsets[0] % 4 == 0
    if ok128:
        modes.insert(0, g.SGEMM_ACCESS_BUFFER_128)
    if variant is not None and g.sgemm_variant_builds(variant) & g.SGEMM_BUILD_BUFFER_128_AB:
        modes.insert(1 if ok128 else 0, g.SGEMM_ACCESS_BUFFER_128_AB)
    return modes
