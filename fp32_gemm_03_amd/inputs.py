"""Seeded synthetic SGEMM inputs, shared by the GPU path's tests and the oracle's.

This module only draws numbers and lays them out; it does no part of the
matrix product.  Every workload is a named problem with its sizes, value
distribution and seed:

* draws come from ``torch.Generator('cpu').manual_seed(seed)`` in float32, in
  the order A (M x K), then B (K x N), then C (M x N) when C is pre-filled;
* ``u01`` is ``torch.rand`` (uniform on [0, 1)), ``upm1`` is
  ``2 * torch.rand - 1`` (uniform on [-1, 1)), ``normal`` is ``torch.randn``;
* ``ones_twos`` is the closed-form case of "3.3 Shared memory ו tiling תרגול",
  section "הכנה" (preparation): A filled with 1.0 and B with 2.0, so every
  element of A @ B equals 2K;
* matrices are row-major with tight leading dimensions (lda = K, ldb = N,
  ldc = N) unless a caller asks for wider ones, in which case the pad columns
  hold a sentinel value (NaN by default) that the product must never touch.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str                   # "u01" | "upm1" | "normal" | "ones_twos"
    seed: int
    alpha: float = 1.0
    beta: float = 0.0
    c_fill: Optional[str] = None  # None: C starts at zero; else a dist name
    note: str = ""

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> float:
        """Each input read once, C written once, and C read once more when beta != 0."""
        c_passes = 2 if self.beta != 0 else 1
        return 4.0 * (self.M * self.K + self.K * self.N + c_passes * self.M * self.N)


WORKLOADS = {w.name: w for w in [
    Workload("square256_u01", 256, 256, 256, "u01", 0,
             note="small square, uniform [0,1)"),
    Workload("square256_closed_form", 256, 256, 256, "ones_twos", 0,
             note="A = 1, B = 2: every C element is exactly 2K = 512"),
    Workload("square4096_upm1", 4096, 4096, 4096, "upm1", 1,
             note="square 4096, uniform [-1,1)"),
    Workload("ragged_1000x1023x999", 1000, 1023, 999, "upm1", 2, 1.5, -0.5, "upm1",
             note="partial tiles on every edge, C pre-filled, beta epilogue"),
    Workload("square1024_normal", 1024, 1024, 1024, "normal", 3),
    Workload("square2048_normal", 2048, 2048, 2048, "normal", 3),
    Workload("square8192_normal", 8192, 8192, 8192, "normal", 3),
    Workload("square16384_normal", 16384, 16384, 16384, "normal", 3),
    Workload("lowk_16384x16384x128", 16384, 16384, 128, "u01", 4, 1.0, 1.0, "u01",
             note="low K, C pre-filled, alpha = beta = 1"),
]}


def _draw(gen: torch.Generator, dist: str, shape) -> torch.Tensor:
    if dist == "u01":
        return torch.rand(shape, generator=gen, dtype=torch.float32)
    if dist == "upm1":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    if dist == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def _embed(mat: torch.Tensor, ld: int, sentinel: float) -> torch.Tensor:
    """Place a rows x cols matrix in a buffer of leading dimension ``ld`` (pad = sentinel)."""
    rows, cols = mat.shape
    if ld == cols:
        return mat.contiguous()
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    buf = torch.full((rows, ld), sentinel, dtype=torch.float32)
    buf[:, :cols] = mat
    return buf


@dataclass
class Problem:
    """Host (CPU, float32) buffers of one SGEMM problem, row-major with leading dims."""
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    A: torch.Tensor      # (M, lda)
    B: torch.Tensor      # (K, ldb)
    C: torch.Tensor      # (M, ldc) -- initial C
    lda: int
    ldb: int
    ldc: int
    name: str = ""
    meta: dict = field(default_factory=dict)

    def np(self, which: str) -> np.ndarray:
        """Flat C-contiguous float32 view of A, B or C (for the oracle)."""
        return getattr(self, which).contiguous().numpy().reshape(-1)


def make_problem(M, N, K, dist="u01", seed=0, alpha=1.0, beta=0.0, c_fill=None,
                 lda=None, ldb=None, ldc=None, sentinel=float("nan"),
                 name="", with_c=True) -> Problem:
    """Draw one problem; see the module docstring for the recipe.  With
    ``with_c=False`` no host C is made (``C`` is an empty tensor): for problems
    whose C is built on the device by the caller."""
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    if dist == "ones_twos":
        a = torch.ones((M, K), dtype=torch.float32)
        b = torch.full((K, N), 2.0, dtype=torch.float32)
    else:
        a = _draw(gen, dist, (M, K))
        b = _draw(gen, dist, (K, N))
    if not with_c:
        c = None
    elif c_fill is None:
        c = torch.zeros((M, N), dtype=torch.float32)
    elif c_fill == "nan":
        c = torch.full((M, N), float("nan"), dtype=torch.float32)
    else:
        c = _draw(gen, c_fill, (M, N))
    lda, ldb, ldc = max(lda, 1), max(ldb, 1), max(ldc, 1)
    return Problem(M, N, K, float(alpha), float(beta),
                   _embed(a, lda, sentinel), _embed(b, ldb, sentinel),
                   torch.empty((0,), dtype=torch.float32) if c is None else _embed(c, ldc, sentinel),
                   lda, ldb, ldc, name=name)


def workload_problem(name: str, **overrides) -> Problem:
    w = WORKLOADS[name]
    kw = dict(M=w.M, N=w.N, K=w.K, dist=w.dist, seed=w.seed, alpha=w.alpha,
              beta=w.beta, c_fill=w.c_fill, name=w.name)
    kw.update(overrides)
    return make_problem(**kw)


def sample_points(M: int, N: int, n_random: int, seed: int, n_lines: int = 4):
    """Seeded (rows, cols) sample: first/last rows and columns, a few seeded full
    rows and columns' worth of points, and ``n_random`` uniform points.

    Returns two int32 vectors.  Edges are always included so that every partial
    tile on the right and bottom is sampled.
    """
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    line_rows = sorted(set([0, M - 1] + list(rng.integers(0, M, n_lines))))
    line_cols = sorted(set([0, N - 1] + list(rng.integers(0, N, n_lines))))
    # a strided subset of each sampled row / column keeps the count bounded
    col_stride = max(1, N // 512)
    row_stride = max(1, M // 512)
    for r in line_rows:
        cs = np.unique(np.concatenate([np.arange(0, N, col_stride), np.arange(max(0, N - 64), N)]))
        rows.append(np.full(cs.size, r)); cols.append(cs)
    for c in line_cols:
        rs = np.unique(np.concatenate([np.arange(0, M, row_stride), np.arange(max(0, M - 64), M)]))
        rows.append(rs); cols.append(np.full(rs.size, c))
    rows.append(rng.integers(0, M, n_random)); cols.append(rng.integers(0, N, n_random))
    return (np.concatenate(rows).astype(np.int32), np.concatenate(cols).astype(np.int32))
