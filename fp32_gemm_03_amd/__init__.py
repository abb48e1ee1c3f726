"""MI355X (gfx950) FP32 SGEMM: C = alpha*A*B + beta*C on row-major matrices.

A thin Python binding of the C ABI in ``include/sgemm.h``: every function has
the name and argument order of its C counterpart and only marshals arguments.
All arithmetic runs in the HIP kernels of ``libsgemm_mi355x.so``; there is no
CPU fallback, and a missing library raises :class:`LibraryNotBuilt`.

Pointer arguments accept a torch tensor on the GPU (its ``data_ptr()`` is
passed) or a raw device address as an ``int``.  ``stream`` accepts a
``torch.cuda.Stream``, a raw ``hipStream_t`` as an ``int``, or ``None`` for
torch's current stream on the current device.
"""
from __future__ import annotations

import ctypes
import os
import threading

from . import inputs  # noqa: F401  (seeded synthetic inputs; no GPU needed)

__all__ = [
    "SGEMM_PATH_AUTO", "SGEMM_PATH_VALU", "SGEMM_PATH_MFMA",
    "SGEMM_ACCESS_AUTO", "SGEMM_ACCESS_BUFFER_128", "SGEMM_ACCESS_BUFFER_32",
    "SGEMM_ACCESS_CHECKED", "SGEMM_ACCESS_BUFFER_128_AB", "sgemm_variant_access",
    "sgemm_ws", "sgemm_ws_noalloc", "SGEMM_NOALLOC_SCRATCH_BYTES", "sgemm_workspace_size", "sgemm_select_splits", "sgemm_splitk",
    "sgemm_splitk_workspace_size", "sgemm_streamk", "sgemm_streamk_workspace_size",
    "sgemm_select_streamk", "sgemm_ws_plan", "sgemm_select_rows", "sgemm_select_pieces",
    "sgemm_plan_for", "sgemm_plan_pieces_for",
    "sgemm_device_shape", "sgemm_tile_order",
    "SgemmError", "LibraryNotBuilt", "library_path", "load_library",
    "sgemm", "sgemm_path", "sgemm_variant", "sgemm_variant_count",
    "sgemm_variant_name", "sgemm_variant_path", "sgemm_variant_tile", "sgemm_variant_reads_a128",
    "sgemm_select_variant", "sgemm_select_variant_for", "sgemm_operands_load16", "sgemm_variant_builds",
    "SGEMM_BUILD_BUFFER_128", "SGEMM_BUILD_BUFFER_32", "SGEMM_BUILD_CHECKED", "SGEMM_BUILD_BUFFER_128_AB",
    "SGEMM_BUILD_SPLITK", "SGEMM_BUILD_STREAMK", "sgemm_status_string", "variants", "sgemm_device_fp32_peak",
]

SGEMM_PATH_AUTO = 0
SGEMM_PATH_VALU = 1
SGEMM_PATH_MFMA = 2

SGEMM_ACCESS_AUTO = 0
SGEMM_ACCESS_BUFFER_128 = 1
SGEMM_ACCESS_BUFFER_32 = 2
SGEMM_ACCESS_CHECKED = 3
SGEMM_ACCESS_BUFFER_128_AB = 4

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIBNAME = "libsgemm_mi355x.so"
_lock = threading.Lock()
_lib = None


class LibraryNotBuilt(RuntimeError):
    pass


class SgemmError(RuntimeError):
    def __init__(self, status: int, where: str = "sgemm"):
        self.status = status
        super().__init__(f"{where}: status {status}: {sgemm_status_string(status)}")


def library_path() -> str:
    return os.path.join(_PKG, _LIBNAME)


def load_library():
    """Load the in-tree HIP library (``python -m fp32_gemm_03_amd.build`` makes it)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise LibraryNotBuilt(
                f"{path} is missing: build it with `python -m fp32_gemm_03_amd.build` "
                "(hipcc, gfx950); there is no CPU fallback")
        lib = ctypes.CDLL(path)
        i, f, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        gemm_args = [i, i, i, f, vp, i, vp, i, f, vp, i, vp]
        lib.sgemm.argtypes = gemm_args
        lib.sgemm.restype = i
        lib.sgemm_path.argtypes = [i] + gemm_args
        lib.sgemm_path.restype = i
        lib.sgemm_variant.argtypes = [i] + gemm_args
        lib.sgemm_variant.restype = i
        lib.sgemm_variant_access.argtypes = [i, i] + gemm_args
        lib.sgemm_variant_access.restype = i
        ws_args = [i, i, i, f, vp, i, vp, i, f, vp, i, vp, ctypes.c_size_t, vp]
        lib.sgemm_ws.argtypes = ws_args
        lib.sgemm_ws.restype = i
        lib.sgemm_ws_noalloc.argtypes = gemm_args
        lib.sgemm_ws_noalloc.restype = i
        lib.sgemm_splitk.argtypes = [i, i] + ws_args
        lib.sgemm_splitk.restype = i
        lib.sgemm_workspace_size.argtypes = [i, i, i]
        lib.sgemm_workspace_size.restype = ctypes.c_size_t
        lib.sgemm_select_splits.argtypes = [i, i, i]
        lib.sgemm_select_splits.restype = i
        lib.sgemm_splitk_workspace_size.argtypes = [i, i, i, i]
        lib.sgemm_splitk_workspace_size.restype = ctypes.c_size_t
        lib.sgemm_streamk.argtypes = [i, i] + ws_args
        lib.sgemm_streamk.restype = i
        lib.sgemm_streamk_workspace_size.argtypes = [i, i]
        lib.sgemm_streamk_workspace_size.restype = ctypes.c_size_t
        lib.sgemm_select_streamk.argtypes = [i, i, i]
        lib.sgemm_select_streamk.restype = i
        lib.sgemm_select_rows.argtypes = [i, i, i]
        lib.sgemm_select_rows.restype = i
        lib.sgemm_ws_plan.argtypes = [i, i, i, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i)]
        lib.sgemm_ws_plan.restype = i
        lib.sgemm_plan_for.argtypes = [i, i, i, i, i, i] + [ctypes.POINTER(i)] * 4
        lib.sgemm_plan_for.restype = i
        lib.sgemm_plan_pieces_for.argtypes = [i, i, i, i, i, i] + [ctypes.POINTER(i)] * 6
        lib.sgemm_plan_pieces_for.restype = i
        lib.sgemm_select_pieces.argtypes = [i, i, i] + [ctypes.POINTER(i)] * 3
        lib.sgemm_select_pieces.restype = i
        lib.sgemm_device_shape.argtypes = [ctypes.POINTER(i), ctypes.POINTER(i)]
        lib.sgemm_device_shape.restype = i
        lib.sgemm_tile_order.argtypes = [i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
        lib.sgemm_tile_order.restype = i
        lib.sgemm_variant_count.argtypes = []
        lib.sgemm_variant_count.restype = i
        lib.sgemm_variant_name.argtypes = [i]
        lib.sgemm_variant_name.restype = ctypes.c_char_p
        lib.sgemm_variant_path.argtypes = [i]
        lib.sgemm_variant_path.restype = i
        lib.sgemm_variant_tile.argtypes = [i, ctypes.POINTER(i), ctypes.POINTER(i)]
        lib.sgemm_variant_tile.restype = i
        lib.sgemm_variant_reads_a128.argtypes = [i]
        lib.sgemm_variant_reads_a128.restype = i
        lib.sgemm_select_variant.argtypes = [i, i, i, i]
        lib.sgemm_select_variant.restype = i
        lib.sgemm_select_variant_for.argtypes = [i, i, i, i, vp, i, vp, i, vp, i]
        lib.sgemm_select_variant_for.restype = i
        lib.sgemm_variant_builds.argtypes = [i]
        lib.sgemm_variant_builds.restype = i
        lib.sgemm_operands_load16.argtypes = [vp, i, vp, i, vp, i]
        lib.sgemm_operands_load16.restype = i
        lib.sgemm_status_string.argtypes = [i]
        lib.sgemm_status_string.restype = ctypes.c_char_p
        lib.sgemm_device_fp32_peak.argtypes = [i, vp, vp, vp]
        lib.sgemm_device_fp32_peak.restype = i
        _lib = lib
        return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    dp = getattr(x, "data_ptr", None)
    if dp is None:
        raise TypeError(f"expected a tensor or an int device address, got {type(x)!r}")
    if getattr(x, "is_cuda", True) is False:
        raise TypeError("SGEMM operands must live in GPU memory")
    return dp()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _gemm_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream):
    return (int(M), int(N), int(K), float(alpha), _ptr(A), int(lda), _ptr(B), int(ldb),
            float(beta), _ptr(C), int(ldc), _stream(stream))


def _ret(status, where, check):
    if check and status != 0:
        raise SgemmError(status, where)
    return status


def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None, check=True):
    """C = alpha*A*B + beta*C; returns the status (raises on nonzero when ``check``)."""
    lib = load_library()
    return _ret(lib.sgemm(*_gemm_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)),
                "sgemm", check)


def sgemm_path(path, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None, check=True):
    lib = load_library()
    return _ret(lib.sgemm_path(int(path), *_gemm_args(M, N, K, alpha, A, lda, B, ldb, beta,
                                                      C, ldc, stream)), "sgemm_path", check)


def sgemm_variant(variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None,
                  check=True):
    lib = load_library()
    return _ret(lib.sgemm_variant(int(variant), *_gemm_args(M, N, K, alpha, A, lda, B, ldb,
                                                            beta, C, ldc, stream)),
                "sgemm_variant", check)


def sgemm_variant_access(variant, access, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         stream=None, check=True):
    lib = load_library()
    return _ret(lib.sgemm_variant_access(int(variant), int(access),
                                         *_gemm_args(M, N, K, alpha, A, lda, B, ldb, beta, C,
                                                     ldc, stream)),
                "sgemm_variant_access", check)


def _ws_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes, stream):
    ws = _ptr(workspace)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (int(M), int(N), int(K), float(alpha), _ptr(A), int(lda), _ptr(B), int(ldb),
            float(beta), _ptr(C), int(ldc), ws, int(workspace_bytes), _stream(stream))


def sgemm_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace=None, workspace_bytes=None,
             stream=None, check=True):
    """sgemm() that may split K, or share K tiles stream-K, over ``workspace`` (a GPU tensor,
    256-byte aligned, any contents)."""
    lib = load_library()
    return _ret(lib.sgemm_ws(*_ws_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                                       workspace_bytes, stream)), "sgemm_ws", check)


SGEMM_NOALLOC_SCRATCH_BYTES = 32 << 20


def sgemm_ws_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None, check=True):
    """sgemm_ws() with its partial tiles in the library's static device scratch (no
    workspace, no allocation); SGEMM_ERR_SCRATCH (-27) when the plan needs more."""
    lib = load_library()
    return _ret(lib.sgemm_ws_noalloc(*_gemm_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)),
                "sgemm_ws_noalloc", check)


def sgemm_splitk(variant, splits, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace=None,
                 workspace_bytes=None, stream=None, check=True):
    lib = load_library()
    return _ret(lib.sgemm_splitk(int(variant), int(splits),
                                 *_ws_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                                           workspace_bytes, stream)), "sgemm_splitk", check)


def sgemm_streamk(variant, workers, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace=None,
                  workspace_bytes=None, stream=None, check=True):
    lib = load_library()
    return _ret(lib.sgemm_streamk(int(variant), int(workers),
                                  *_ws_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                                            workspace_bytes, stream)), "sgemm_streamk", check)


def sgemm_streamk_workspace_size(variant, workers) -> int:
    return int(load_library().sgemm_streamk_workspace_size(int(variant), int(workers)))


def sgemm_select_streamk(M, N, K) -> int:
    return int(load_library().sgemm_select_streamk(int(M), int(N), int(K)))


def sgemm_select_rows(M, N, K) -> int:
    """Rows of the first piece ``sgemm`` cuts C into (0: one launch)."""
    return int(load_library().sgemm_select_rows(int(M), int(N), int(K)))


def sgemm_select_pieces(M, N, K):
    """``(status, rows, cols, first_variant)``: the first piece ``sgemm`` cuts C into, rows x
    cols at the top left, and the variant it runs on (rows 0: one launch; cols == N: a cut by
    rows alone)."""
    r, c, v = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(-1)
    rc = load_library().sgemm_select_pieces(int(M), int(N), int(K), ctypes.byref(r), ctypes.byref(c),
                                            ctypes.byref(v))
    return int(rc), r.value, c.value, v.value


def sgemm_ws_plan(M, N, K):
    """``(status, variant, splits, workers)``: what sgemm_ws() runs with enough workspace."""
    v, sp, w = ctypes.c_int(-1), ctypes.c_int(0), ctypes.c_int(0)
    rc = load_library().sgemm_ws_plan(int(M), int(N), int(K), ctypes.byref(v), ctypes.byref(sp),
                                      ctypes.byref(w))
    return int(rc), v.value, sp.value, w.value


def sgemm_plan_for(compute_units, M, N, K, with_workspace=False, operands_load16=True):
    """``(status, variant, splits, workers, rows)``: the plan for these sizes on a device of
    ``compute_units`` CUs (``sgemm_ws`` with enough workspace, or ``sgemm`` without), for
    operands that allow 16-byte loads of A and B or (``operands_load16=False``) others."""
    v, sp, w, r = ctypes.c_int(-1), ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    rc = load_library().sgemm_plan_for(int(compute_units), int(M), int(N), int(K),
                                       1 if with_workspace else 0, 1 if operands_load16 else 0,
                                       ctypes.byref(v), ctypes.byref(sp), ctypes.byref(w),
                                       ctypes.byref(r))
    return int(rc), v.value, sp.value, w.value, r.value


def sgemm_plan_pieces_for(compute_units, M, N, K, with_workspace=False, operands_load16=True):
    """``sgemm_plan_for`` with the first piece's columns and variant: ``(status, variant,
    splits, workers, rows, cols, first_variant)``."""
    v, sp, w = ctypes.c_int(-1), ctypes.c_int(0), ctypes.c_int(0)
    r, c, fv = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(-1)
    rc = load_library().sgemm_plan_pieces_for(int(compute_units), int(M), int(N), int(K),
                                              1 if with_workspace else 0, 1 if operands_load16 else 0,
                                              ctypes.byref(v), ctypes.byref(sp), ctypes.byref(w),
                                              ctypes.byref(r), ctypes.byref(c), ctypes.byref(fv))
    return int(rc), v.value, sp.value, w.value, r.value, c.value, fv.value


def sgemm_device_shape():
    """``(compute_units, xcds)`` the current device's choices use."""
    cu, x = ctypes.c_int(0), ctypes.c_int(0)
    load_library().sgemm_device_shape(ctypes.byref(cu), ctypes.byref(x))
    return cu.value, x.value


def sgemm_tile_order(xcds, nbm, nbn):
    """``(status, tile_m, tile_n)``: the tile each workgroup of an nbm x nbn grid computes."""
    n = max(int(nbm) * int(nbn), 0)
    tm = (ctypes.c_int * max(n, 1))()
    tn = (ctypes.c_int * max(n, 1))()
    rc = load_library().sgemm_tile_order(int(xcds), int(nbm), int(nbn), tm, tn)
    return int(rc), list(tm)[:n], list(tn)[:n]


def variant_has_streamk(variant) -> bool:
    """True when the variant's split builds also run stream-K."""
    return sgemm_streamk_workspace_size(variant, 256) > 0


def sgemm_workspace_size(M, N, K) -> int:
    return int(load_library().sgemm_workspace_size(int(M), int(N), int(K)))


def sgemm_select_splits(M, N, K) -> int:
    return int(load_library().sgemm_select_splits(int(M), int(N), int(K)))


def sgemm_splitk_workspace_size(variant, splits, M, N) -> int:
    return int(load_library().sgemm_splitk_workspace_size(int(variant), int(splits), int(M), int(N)))


def variant_has_splitk(variant) -> bool:
    """True when the variant has a split-K build (workspace size > 0 for 2 splits)."""
    return sgemm_splitk_workspace_size(variant, 2, 64, 64) > 0


def sgemm_variant_count() -> int:
    return int(load_library().sgemm_variant_count())


SGEMM_BUILD_BUFFER_128, SGEMM_BUILD_BUFFER_32, SGEMM_BUILD_CHECKED = 1, 2, 4
SGEMM_BUILD_BUFFER_128_AB, SGEMM_BUILD_SPLITK, SGEMM_BUILD_STREAMK = 8, 16, 32


def sgemm_variant_builds(variant) -> int:
    """Bit mask of the builds a variant has (SGEMM_BUILD_*), or SGEMM_ERR_VARIANT."""
    return int(load_library().sgemm_variant_builds(int(variant)))


def sgemm_variant_name(variant):
    r = load_library().sgemm_variant_name(int(variant))
    return None if r is None else r.decode()


def sgemm_variant_path(variant) -> int:
    return int(load_library().sgemm_variant_path(int(variant)))


def sgemm_variant_tile(variant):
    """``(status, bm, bn)``."""
    bm, bn = ctypes.c_int(0), ctypes.c_int(0)
    rc = load_library().sgemm_variant_tile(int(variant), ctypes.byref(bm), ctypes.byref(bn))
    return int(rc), bm.value, bn.value


def sgemm_variant_reads_a128(variant) -> int:
    """1 if the variant's 128-bit build also reads A 128 bits at a time along K, else 0."""
    return int(load_library().sgemm_variant_reads_a128(int(variant)))


def sgemm_select_variant(path, M, N, K) -> int:
    return int(load_library().sgemm_select_variant(int(path), int(M), int(N), int(K)))


def sgemm_operands_load16(A, lda, B, ldb, C, ldc) -> bool:
    """True when these operands allow 16-byte loads of A and B (4-byte aligned bases, leading
    dimensions below about 2^24): the small blocks, split-K and stream-K need them."""
    return bool(load_library().sgemm_operands_load16(_ptr(A), int(lda), _ptr(B), int(ldb),
                                                     _ptr(C), int(ldc)))


def sgemm_select_variant_for(path, M, N, K, A, lda, B, ldb, C, ldc) -> int:
    """The variant sgemm_path() launches for these operands (their alignment decides)."""
    return int(load_library().sgemm_select_variant_for(int(path), int(M), int(N), int(K), _ptr(A),
                                                       int(lda), _ptr(B), int(ldb), _ptr(C), int(ldc)))


def sgemm_status_string(status) -> str:
    return load_library().sgemm_status_string(int(status)).decode()


def sgemm_device_fp32_peak(device=0):
    """``(compute_units, clock_khz, tflops)`` of a device from its properties."""
    lib = load_library()
    cu, clk, tf = ctypes.c_int(), ctypes.c_int(), ctypes.c_double()
    st = lib.sgemm_device_fp32_peak(int(device), ctypes.byref(cu), ctypes.byref(clk), ctypes.byref(tf))
    if st != 0:
        raise SgemmError(st, "sgemm_device_fp32_peak")
    return cu.value, clk.value, tf.value


def variants():
    """``[(index, name, path, bm, bn), ...]`` for every compiled variant."""
    out = []
    for v in range(sgemm_variant_count()):
        _, bm, bn = sgemm_variant_tile(v)
        out.append((v, sgemm_variant_name(v), sgemm_variant_path(v), bm, bn))
    return out
