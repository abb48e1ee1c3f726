"""Pins of the float64 SGEMM oracle to facts outside the oracle itself.

Each ``pin_*`` function takes an oracle front end (``oracle.OracleLib``) and
raises ``AssertionError`` when that oracle disagrees with:

* the closed form of "3.3 Shared memory ו tiling תרגול", section "הכנה"
  (A = 1, B = 2 gives every element of C equal to 2K), values stored in
  ``tests/golden/closed_form.txt``;
* exact rational arithmetic (``fractions.Fraction``) on tiny shapes, with wide
  leading dimensions whose pad columns hold NaN;
* numpy's float64 ``matmul`` of the up-cast inputs (a library routine);
* invariants of the definition: identity, K = 1, power-of-two alpha, alpha = 0
  with NaN and Inf in A and B (A and B not read), beta = 0 with NaN in C (C
  not read), transposition, and that the two entry
  points, every thread count and every row band give the same sums bit for bit.

They are run against the real oracle by ``test_oracle.py`` and against
deliberately broken copies of it by ``test_oracle_mutants.py``.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = 2.0 ** -53  # unit roundoff of float64


def read_closed_form():
    rows = []
    with open(os.path.join(GOLDEN, "closed_form.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            M, N, K, a, b, e = line.split()
            rows.append((int(M), int(N), int(K), float(a), float(b), float(e)))
    return rows


def _nan_c(M, N):
    """C for beta = 0 calls: all NaN, which must never be read."""
    return np.full(max(M * N, 1), np.nan, dtype=np.float32)


def _padded(rng, rows, cols, ld, lo=-1.0, hi=1.0):
    """Random float32 matrix in a buffer of leading dimension ld; pad columns are NaN."""
    buf = np.full((rows, ld), np.nan, dtype=np.float32)
    buf[:, :cols] = rng.uniform(lo, hi, size=(rows, cols)).astype(np.float32)
    return buf.reshape(-1)


def _exact(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    """Exact rational value and denominator of the pass rule at every element."""
    out = np.empty((M, N), dtype=object)
    den = np.empty((M, N), dtype=object)
    fa, fb = Fraction(float(np.float32(alpha))), Fraction(float(np.float32(beta)))
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            sa = Fraction(0)
            for k in range(K):
                p = Fraction(float(A[i * lda + k])) * Fraction(float(B[k * ldb + j]))
                s += p
                sa += abs(p)
            v = fa * s
            d = abs(fa) * sa
            if beta != 0:
                c = Fraction(float(C[i * ldc + j]))
                v += fb * c
                d += abs(fb) * abs(c)
            out[i, j] = v
            den[i, j] = d
    return out, den


# ---------------------------------------------------------------- closed form
def pin_closed_form(api, max_n=None):
    for M, N, K, a, b, expected in read_closed_form():
        if max_n is not None and max(M, N, K) > max_n:
            continue
        A = np.full(M * K, a, dtype=np.float32)
        B = np.full(K * N, b, dtype=np.float32)
        C = np.full(M * N, np.nan, dtype=np.float32)   # beta = 0: never read
        ref, den = api.sgemm(M, N, K, 1.0, A, K, B, N, 0.0, C, N)
        assert np.all(ref == expected), (M, N, K, np.unique(ref)[:5])
        assert np.all(np.abs(den - expected) <= 1e-29), "denominator of all-positive data"


# ---------------------------------------------------------------- brute force
BRUTE_SHAPES = [(m, n, k) for m in (1, 2, 3, 5) for n in (1, 2, 4, 6) for k in (1, 2, 3, 6)] + [
    (7, 9, 11), (13, 5, 17), (17, 16, 15), (4, 17, 9), (16, 1, 13)]
BRUTE_SCALARS = [(1.0, 0.0), (1.5, -0.5), (-2.0, 1.0), (0.3, 2.0), (0.0, 1.5), (1.0, 1.0)]


def pin_bruteforce(api, shapes=BRUTE_SHAPES, seed=1234):
    rng = np.random.default_rng(seed)
    for idx, (M, N, K) in enumerate(shapes):
        alpha, beta = BRUTE_SCALARS[idx % len(BRUTE_SCALARS)]
        lda, ldb, ldc = K + (idx % 3), N + (idx % 2), N + ((idx + 1) % 3)
        A = _padded(rng, M, K, lda)
        B = _padded(rng, K, N, ldb)
        C = _padded(rng, M, N, ldc)
        exact, exact_den = _exact(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
        ref, den = api.sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
        rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        pref, pden = api.sgemm_points(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                      rows.reshape(-1), cols.reshape(-1))
        for name, r, d in (("rows", ref, den), ("points", pref.reshape(M, N), pden.reshape(M, N))):
            for i in range(M):
                for j in range(N):
                    ex, exd = exact[i, j], exact_den[i, j]
                    tol = (K + 4) * U * float(exd) * 1.01
                    assert np.isfinite(r[i, j]) and np.isfinite(d[i, j]), (name, M, N, K, i, j)
                    assert abs(Fraction(float(r[i, j])) - ex) <= Fraction(tol) + Fraction(1, 10 ** 300), \
                        (name, M, N, K, alpha, beta, i, j, float(r[i, j]), float(ex))
                    assert abs(float(d[i, j]) - 1e-30 - float(exd)) <= tol + 1e-30, \
                        (name, "den", M, N, K, i, j, float(d[i, j]), float(exd))


# ---------------------------------------------------------------- library routine
def pin_numpy(api, shapes=((96, 80, 72), (130, 257, 129)), seed=7):
    rng = np.random.default_rng(seed)
    for M, N, K in shapes:
        for alpha, beta in ((1.0, 0.0), (1.5, -0.5)):
            A = rng.standard_normal(M * K).astype(np.float32)
            B = rng.standard_normal(K * N).astype(np.float32)
            C = rng.standard_normal(M * N).astype(np.float32)
            ref, den = api.sgemm(M, N, K, alpha, A, K, B, N, beta, C, N)
            A64 = A.reshape(M, K).astype(np.float64)
            B64 = B.reshape(K, N).astype(np.float64)
            C64 = C.reshape(M, N).astype(np.float64)
            want = np.float64(np.float32(alpha)) * (A64 @ B64)
            want_den = abs(np.float64(np.float32(alpha))) * (np.abs(A64) @ np.abs(B64))
            if beta != 0:
                want = want + np.float64(np.float32(beta)) * C64
                want_den = want_den + abs(np.float64(np.float32(beta))) * np.abs(C64)
            assert np.max(np.abs(ref - want) / den) <= 1e-12, (M, N, K, alpha, beta)
            assert np.max(np.abs(den - 1e-30 - want_den) / den) <= 1e-12, (M, N, K, "den")


# ---------------------------------------------------------------- invariants
def pin_invariants(api, seed=99):
    rng = np.random.default_rng(seed)

    # identity: A = I (M = K) gives alpha*B exactly when alpha is a power of two
    n, N = 24, 19
    A = np.eye(n, dtype=np.float32).reshape(-1)
    B = rng.standard_normal(n * N).astype(np.float32)
    ref, _ = api.sgemm(n, N, n, 1.0, A, n, B, N, 0.0, _nan_c(n, N), N)
    assert np.array_equal(ref, B.reshape(n, N).astype(np.float64)), "identity"
    ref, _ = api.sgemm(n, N, n, -4.0, A, n, B, N, 0.0, _nan_c(n, N), N)
    assert np.array_equal(ref, -4.0 * B.reshape(n, N).astype(np.float64)), "identity, alpha=-4"

    # K = 1: the outer product, each element one exact product
    M, N = 11, 13
    a = rng.standard_normal(M).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    ref, _ = api.sgemm(M, N, 1, 1.0, a, 1, b, N, 0.0, _nan_c(M, N), N)
    assert np.array_equal(ref, np.outer(a.astype(np.float64), b.astype(np.float64))), "K=1"

    # power-of-two alpha scales bit for bit; alpha = 0 leaves beta*C exactly
    M, N, K = 9, 10, 33
    A = rng.standard_normal(M * K).astype(np.float32)
    B = rng.standard_normal(K * N).astype(np.float32)
    C = rng.standard_normal(M * N).astype(np.float32)
    r1, d1 = api.sgemm(M, N, K, 1.0, A, K, B, N, 0.0, _nan_c(M, N), N)
    r8, d8 = api.sgemm(M, N, K, 8.0, A, K, B, N, 0.0, _nan_c(M, N), N)
    assert np.array_equal(r8, 8.0 * r1), "alpha = 8"
    assert np.array_equal(d8 - 1e-30, 8.0 * (d1 - 1e-30)), "alpha = 8, den"
    r0, _ = api.sgemm(M, N, K, 0.0, A, K, B, N, -0.5, C, N)
    assert np.array_equal(r0, -0.5 * C.reshape(M, N).astype(np.float64)), "alpha = 0"

    # alpha = 0: A and B are not read, so NaN and Inf in them do not reach the
    # result, which is beta*C exactly (0 with beta = 0), in both entry points
    Abad = np.where(np.arange(M * K) % 2 == 0, np.nan, np.inf).astype(np.float32)
    Bbad = np.full(K * N, np.nan, dtype=np.float32)
    want = -0.5 * C.reshape(M, N).astype(np.float64)
    want_den = 0.5 * np.abs(C.reshape(M, N).astype(np.float64)) + 1e-30
    rz, dz = api.sgemm(M, N, K, 0.0, Abad, K, Bbad, N, -0.5, C, N)
    assert np.array_equal(rz, want) and np.array_equal(dz, want_den), "alpha = 0, NaN A and B"
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    pz, pdz = api.sgemm_points(M, N, K, 0.0, Abad, K, Bbad, N, -0.5, C, N,
                               rows.reshape(-1), cols.reshape(-1))
    assert np.array_equal(pz.reshape(M, N), want) and np.array_equal(pdz.reshape(M, N), want_den), \
        "alpha = 0, NaN A and B, points"
    rzz, _ = api.sgemm(M, N, K, 0.0, Abad, K, Bbad, N, 0.0, _nan_c(M, N), N)
    assert np.all(rzz == 0.0), "alpha = beta = 0 with NaN everywhere"

    # beta = 0: C is not read, so NaN in C does not reach the result
    Cnan = np.full(M * N, np.nan, dtype=np.float32)
    rn, dn = api.sgemm(M, N, K, 1.0, A, K, B, N, 0.0, Cnan, N)
    assert np.array_equal(rn, r1) and np.array_equal(dn, d1), "beta = 0 with NaN C"

    # beta = 1, alpha = 1 adds C exactly once
    r11, _ = api.sgemm(M, N, K, 1.0, A, K, B, N, 1.0, C, N)
    assert np.array_equal(r11, r1 + C.reshape(M, N).astype(np.float64)), "beta = 1"

    # transposition: (A B)^T = B^T A^T, the same products summed in the same order
    M, N, K = 7, 12, 21
    A = rng.standard_normal(M * K).astype(np.float32)
    B = rng.standard_normal(K * N).astype(np.float32)
    AT = np.ascontiguousarray(A.reshape(M, K).T).reshape(-1)
    BT = np.ascontiguousarray(B.reshape(K, N).T).reshape(-1)
    r, d = api.sgemm(M, N, K, 1.0, A, K, B, N, 0.0, _nan_c(M, N), N)
    rt, dt = api.sgemm(N, M, K, 1.0, BT, K, AT, M, 0.0, _nan_c(N, M), M)
    assert np.array_equal(r, rt.T) and np.array_equal(d, dt.T), "transposition"

    # row entry vs point entry, thread counts, row bands: identical sums
    M, N, K = 37, 29, 45
    A = rng.standard_normal(M * K).astype(np.float32)
    B = rng.standard_normal(K * N).astype(np.float32)
    C = rng.standard_normal(M * N).astype(np.float32)
    full, fden = api.sgemm_rows(M, N, K, 1.25, A, K, B, N, 0.75, C, N, nthreads=1)
    for t in (2, 3, 8):
        f2, d2 = api.sgemm_rows(M, N, K, 1.25, A, K, B, N, 0.75, C, N, nthreads=t)
        assert np.array_equal(full, f2) and np.array_equal(fden, d2), f"nthreads={t}"
    band, bden = api.sgemm_rows(M, N, K, 1.25, A, K, B, N, 0.75, C, N, row0=10, nrows=9)
    assert np.array_equal(band, full[10:19]) and np.array_equal(bden, fden[10:19]), "row band"
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    pr, pd = api.sgemm_points(M, N, K, 1.25, A, K, B, N, 0.75, C, N,
                              rows.reshape(-1), cols.reshape(-1))
    assert np.array_equal(pr.reshape(M, N), full) and np.array_equal(pd.reshape(M, N), fden), \
        "rows vs points"


QUICK_PINS = (
    ("closed_form", lambda api: pin_closed_form(api, max_n=256)),
    ("bruteforce", pin_bruteforce),
    ("numpy", lambda api: pin_numpy(api, shapes=((40, 33, 27),))),
    ("invariants", pin_invariants),
)
