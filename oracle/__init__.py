"""CPU float64 oracle for SGEMM -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never imports, links or calls it, and it
imports nothing from the GPU library.

It wraps ``oracle_sgemm.c`` (plain C, float64 sums, POSIX threads), which
follows the plain definition of the naive GEMM in "如何高效实现矩阵乘？CUDA初学者的
角度入门", section "樸素 GEMM 與前置知識": C = alpha * (A @ B) + beta * C on
row-major matrices, alpha applied once to the finished dot product.  With
beta == 0 the input C is not read; with alpha == 0 neither A nor B is read
(the product term is dropped, so the result is beta * C exactly).

The pass rule used against it is ``max |C_gpu - ref| / den``, with
``den = |alpha| * sum_k |A_ik||B_kj| + |beta||C_ij| + 1e-30``; see
:func:`max_error_ratio`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle_sgemm.c")
LIBRARY = os.path.join(_HERE, "liboracle_sgemm.so")

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int)


def compile_c(source: str, out: str) -> str:
    """gcc a C file of this package's shape into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle_sgemm.so``."""
    if force or not os.path.exists(LIBRARY):
        compile_c(SOURCE, LIBRARY)
    return LIBRARY


def _fptr(a):
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype != np.float32 or not a.flags["C_CONTIGUOUS"]:
        raise TypeError("oracle buffers must be C-contiguous float32 arrays")
    return a.ctypes.data_as(_f32p)


def _check_extent(name, buf, rows, cols, ld):
    """The buffer must hold element (rows-1, cols-1) at (rows-1)*ld + cols-1."""
    if buf is None or rows == 0 or cols == 0:
        return
    need = (rows - 1) * ld + cols
    if np.asarray(buf).size < need:
        raise ValueError(f"{name}: buffer of {np.asarray(buf).size} floats, "
                         f"{rows}x{cols} with ld={ld} needs {need}")


class OracleLib:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_sgemm_rows.restype = ctypes.c_int
        lib.oracle_sgemm_rows.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            _f32p, ctypes.c_int, _f32p, ctypes.c_int, ctypes.c_float,
            _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            _f64p, _f64p, ctypes.c_int]
        lib.oracle_sgemm_points.restype = ctypes.c_int
        lib.oracle_sgemm_points.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            _f32p, ctypes.c_int, _f32p, ctypes.c_int, ctypes.c_float,
            _f32p, ctypes.c_int, ctypes.c_int, _i32p, _i32p, _f64p, _f64p]
        lib.oracle_nthreads.restype = ctypes.c_int
        lib.oracle_nthreads.argtypes = []
        self.path = path
        self._lib = lib

    def nthreads(self) -> int:
        """Threads the oracle uses when asked for ``nthreads <= 0`` (online CPUs)."""
        return int(self._lib.oracle_nthreads())

    def sgemm_rows(self, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                   row0=0, nrows=None, nthreads=0):
        """Reference rows ``[row0, row0 + nrows)``: ``(ref, den)``, float64, shape (nrows, N).

        ``A``, ``B``, ``C`` are C-contiguous float32 buffers holding row-major
        matrices with leading dimensions ``lda``, ``ldb``, ``ldc`` (``C`` may
        be ``None`` when ``beta == 0``: it is not read then).
        """
        if nrows is None:
            nrows = M - row0
        _check_extent("A", A, M, K, lda)
        _check_extent("B", B, K, N, ldb)
        if C is not None:
            _check_extent("C", C, M, N, ldc)
        elif beta != 0:
            raise ValueError("C is needed when beta != 0")
        ref = np.empty((nrows, N), dtype=np.float64)
        den = np.empty((nrows, N), dtype=np.float64)
        rc = self._lib.oracle_sgemm_rows(
            M, N, K, float(alpha), _fptr(A), lda, _fptr(B), ldb, float(beta),
            _fptr(C), ldc, row0, nrows,
            ref.ctypes.data_as(_f64p), den.ctypes.data_as(_f64p), int(nthreads))
        if rc != 0:
            raise ValueError(f"oracle_sgemm_rows failed with status {rc}")
        return ref, den

    def sgemm_points(self, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, rows, cols):
        """Reference values at ``(rows[p], cols[p])``: ``(ref, den)`` float64 vectors."""
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        cols = np.ascontiguousarray(cols, dtype=np.int32)
        if rows.shape != cols.shape or rows.ndim != 1:
            raise ValueError("rows and cols must be 1-D and of equal length")
        _check_extent("A", A, M, K, lda)
        _check_extent("B", B, K, N, ldb)
        if C is not None:
            _check_extent("C", C, M, N, ldc)
        elif beta != 0:
            raise ValueError("C is needed when beta != 0")
        n = rows.size
        ref = np.empty(n, dtype=np.float64)
        den = np.empty(n, dtype=np.float64)
        rc = self._lib.oracle_sgemm_points(
            M, N, K, float(alpha), _fptr(A), lda, _fptr(B), ldb, float(beta),
            _fptr(C), ldc, n,
            rows.ctypes.data_as(_i32p), cols.ctypes.data_as(_i32p),
            ref.ctypes.data_as(_f64p), den.ctypes.data_as(_f64p))
        if rc != 0:
            raise ValueError(f"oracle_sgemm_points failed with status {rc}")
        return ref, den

    def sgemm(self, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, nthreads=0):
        """Every element: ``(ref, den)`` of shape (M, N)."""
        return self.sgemm_rows(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                               0, M, nthreads)


_lock = threading.Lock()
_default = None


def default() -> OracleLib:
    """The oracle built from ``oracle_sgemm.c`` (compiled on first use if absent)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIBRARY):
                build(force=False)
            _default = OracleLib(LIBRARY)
    return _default


def nthreads() -> int:
    return default().nthreads()


def sgemm_rows(*args, **kwargs):
    return default().sgemm_rows(*args, **kwargs)


def sgemm_points(*args, **kwargs):
    return default().sgemm_points(*args, **kwargs)


def sgemm(*args, **kwargs):
    return default().sgemm(*args, **kwargs)


def max_error_ratio(c, ref, den) -> float:
    """``max |c - ref| / den`` over all elements (float64); NaN anywhere gives inf.

    The pass rule for a float32 result against the oracle is
    ``max_error_ratio(...) <= 1e-5``.
    """
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    if c.shape != ref.shape or ref.shape != den.shape:
        raise ValueError(f"shape mismatch {c.shape} {ref.shape} {den.shape}")
    if c.size == 0:
        return 0.0
    err = np.abs(c - ref) / den
    if not np.all(np.isfinite(err)):
        return float("inf")
    return float(err.max())
