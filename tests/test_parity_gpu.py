"""GPU parity: the HIP library, called through its C ABI, against the float64
oracle on seeded inputs.  Pass rule: max |C_gpu - ref| / den <= 1e-5 with
den = |alpha| sum_k |A_ik||B_kj| + |beta||C_ij| + 1e-30, at every element for
sizes the oracle finishes in seconds, and at seeded samples (first and last
rows and columns, seeded rows and columns, random points) for the full sizes.
Exact cases (closed form, alpha = 0, K = 0) must match bit for bit."""
import functools

import numpy as np
import pytest
import torch

import fp32_gemm_03_amd as g
from fp32_gemm_03_amd import inputs
from tests import gpu_util as gu
import oracle

pytestmark = pytest.mark.gpu

TOL = gu.TOL


def all_variants():
    return list(range(g.sgemm_variant_count()))


ACCESSES = [g.SGEMM_ACCESS_BUFFER_128, g.SGEMM_ACCESS_BUFFER_32, g.SGEMM_ACCESS_CHECKED]


def combos():
    """Every compiled kernel: (variant, access mode)."""
    return [(v, acc) for v in all_variants() for acc in ACCESSES]


def combo_id(c):
    return f"{g.sgemm_variant_name(c[0])}-{gu.ACCESS_NAMES[c[1]]}"


def run_all_modes(p, variant, offsets=(0, 0, 0)):
    """Run every access mode the arguments allow; yields (mode, output)."""
    for acc in gu.allowed_accesses(p, offsets, variant):
        gu.say("  access", gu.ACCESS_NAMES[acc])
        yield acc, gu.run(p, variant=variant, access=acc, offsets=offsets)


@functools.lru_cache(maxsize=None)
def cached_problem(name):
    return inputs.workload_problem(name)


@functools.lru_cache(maxsize=None)
def cached_oracle(name):
    return gu.oracle_full(cached_problem(name))


@pytest.fixture(autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ------------------------------------------------------------------ exact cases
@pytest.mark.parametrize("variant", all_variants())
def test_closed_form_every_variant(variant):
    p = cached_problem("square256_closed_form")
    gu.say("closed form 256^3", g.sgemm_variant_name(variant))
    for acc, out in run_all_modes(p, variant):
        assert np.all(out == 512.0), (acc, np.unique(out)[:8])


@pytest.mark.parametrize("variant", all_variants())
def test_closed_form_nonsquare_ragged(variant):
    # every element is exactly 2K for any shape, including partial tiles
    for M, N, K in [(131, 77, 203), (131, 80, 203)]:
        p = inputs.make_problem(M, N, K, dist="ones_twos")
        gu.say("closed form", M, N, K, g.sgemm_variant_name(variant))
        for acc, out in run_all_modes(p, variant):
            assert np.all(out == 2.0 * K), (M, N, K, acc)


@pytest.mark.parametrize("variant", all_variants())
def test_alpha_zero_and_k_zero_give_beta_c(variant):
    p = inputs.make_problem(70, 45, 33, dist="upm1", seed=5, alpha=0.0, beta=-0.5, c_fill="upm1")
    gu.say("alpha=0", g.sgemm_variant_name(variant))
    for acc, out in run_all_modes(p, variant):
        assert np.array_equal(out, (np.float32(-0.5) * p.C.numpy())), acc
    p0 = inputs.make_problem(70, 45, 0, dist="upm1", seed=5, alpha=1.0, beta=2.0, c_fill="upm1")
    gu.say("K=0", g.sgemm_variant_name(variant))
    for acc, out in run_all_modes(p0, variant):
        assert np.array_equal(out, (np.float32(2.0) * p0.C.numpy())), acc
    pz = inputs.make_problem(70, 48, 0, dist="upm1", seed=5, beta=0.0, c_fill="nan")
    gu.say("K=0 beta=0", g.sgemm_variant_name(variant))
    for acc, out in run_all_modes(pz, variant):
        assert np.all(out == 0.0), acc


@pytest.mark.parametrize("variant", all_variants())
def test_alpha_zero_reads_neither_a_nor_b(variant):
    """alpha = 0: A and B are not read, so NaN and Inf in them do not reach C,
    which is beta*C exactly (0 with beta = 0, even over NaN in C), as the
    oracle reads it too."""
    p = inputs.make_problem(70, 48, 33, dist="upm1", seed=6, alpha=0.0, beta=-0.5, c_fill="upm1")
    p.A[:, ::2] = float("nan")
    p.A[:, 1::2] = float("inf")
    p.B[:] = float("nan")
    ref, den = gu.oracle_full(p)
    assert np.array_equal(ref, np.float64(-0.5) * p.C.numpy().astype(np.float64))
    gu.say("alpha=0 NaN/Inf A, B", g.sgemm_variant_name(variant))
    for acc, out in run_all_modes(p, variant):
        assert np.array_equal(out, np.float32(-0.5) * p.C.numpy()), acc
        assert gu.ratio_full(p, out, (ref, den)) == 0.0, acc
    pz = inputs.make_problem(70, 48, 33, dist="upm1", seed=6, alpha=0.0, beta=0.0, c_fill="nan")
    pz.A[:] = float("nan")
    pz.B[:] = float("inf")
    for acc, out in run_all_modes(pz, variant):
        assert np.all(out == 0.0), acc


# ------------------------------------------------------------------ workloads, every element
@pytest.mark.parametrize("name", ["square256_u01", "ragged_1000x1023x999", "square1024_normal"])
@pytest.mark.parametrize("variant", all_variants())
def test_workloads_every_variant(name, variant):
    p = cached_problem(name)
    gu.say(name, g.sgemm_variant_name(variant))
    for acc, out in run_all_modes(p, variant):
        r = gu.ratio_full(p, out, cached_oracle(name))
        assert r <= TOL, (name, g.sgemm_variant_name(variant), acc, r)


def test_forced_access_mode_preconditions():
    # 128-bit accesses are refused when B or C cannot take them
    p = inputs.make_problem(64, 63, 32, dist="upm1", seed=1)
    _, _, a = gu.to_gpu(p.A)
    _, _, b = gu.to_gpu(p.B)
    oc, _, c = gu.to_gpu(p.C)
    rc = g.sgemm_variant_access(1, g.SGEMM_ACCESS_BUFFER_128, p.M, p.N, p.K, 1.0, a, p.lda, b,
                                p.ldb, 0.0, c, p.ldc, check=False)
    assert rc == -23
    rc = g.sgemm_variant_access(1, 7, p.M, p.N, p.K, 1.0, a, p.lda, b, p.ldb, 0.0, c, p.ldc,
                                check=False)
    assert rc == -23
    torch.cuda.synchronize()
    del oc


@pytest.mark.parametrize("name", ["square256_u01", "ragged_1000x1023x999", "square1024_normal"])
@pytest.mark.parametrize("path", [g.SGEMM_PATH_AUTO, g.SGEMM_PATH_VALU, g.SGEMM_PATH_MFMA])
def test_workloads_every_path(name, path):
    p = cached_problem(name)
    gu.say(name, "path", path)
    out = gu.run(p, path=path)
    assert gu.ratio_full(p, out, cached_oracle(name)) <= TOL


# ------------------------------------------------------------------ edges
EDGE = [1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257]


def edge_shapes():
    rng = np.random.default_rng(2024)
    shapes = [(e, e, e) for e in EDGE]
    for _ in range(40):
        shapes.append(tuple(int(x) for x in rng.choice(EDGE, 3)))
    shapes += [(1, 300, 7), (300, 1, 7), (5, 5, 513), (257, 129, 1), (96, 260, 35)]
    return shapes


SCALARS = [(1.0, 0.0), (1.5, -0.5), (-1.0, 1.0), (2.0, 1.5), (0.5, 2.0)]


@pytest.mark.parametrize("variant", all_variants())
def test_edge_sweep(variant):
    for idx, (M, N, K) in enumerate(edge_shapes()):
        alpha, beta = SCALARS[idx % len(SCALARS)]
        p = inputs.make_problem(M, N, K, dist="upm1", seed=idx, alpha=alpha, beta=beta,
                                c_fill="upm1" if beta != 0 else None)
        gu.say("edge", M, N, K, alpha, beta, g.sgemm_variant_name(variant))
        ref = gu.oracle_full(p)
        for acc, out in run_all_modes(p, variant):
            r = gu.ratio_full(p, out, ref)
            assert r <= TOL, (M, N, K, alpha, beta, g.sgemm_variant_name(variant), acc, r)


@pytest.mark.parametrize("variant", all_variants())
@pytest.mark.parametrize("offsets", [(0, 0, 0), (1, 0, 0), (0, 1, 0), (0, 0, 1), (3, 1, 2)])
def test_wide_leading_dims_and_misaligned_bases(variant, offsets):
    # pad columns of A, B, C hold NaN; they must never be read or written
    # (K % 4 != 0 with lda > K: a 16-byte chunk of A that holds column K - 1
    # brings NaN pad columns along, which must not reach C)
    for (M, N, K, lda, ldb, ldc) in [(130, 196, 72, 75, 200, 204), (97, 64, 40, 41, 67, 66),
                                     (64, 128, 64, 68, 132, 128), (70, 50, 41, 43, 53, 52),
                                     (33, 97, 6, 7, 99, 100)]:
        p = inputs.make_problem(M, N, K, dist="upm1", seed=M + N, alpha=1.25, beta=-0.75,
                                c_fill="upm1", lda=lda, ldb=ldb, ldc=ldc)
        gu.say("wide-ld", M, N, K, lda, ldb, ldc, offsets, g.sgemm_variant_name(variant))
        ref = gu.oracle_full(p)
        for acc, out in run_all_modes(p, variant, offsets):
            assert gu.pad_untouched(p, out), acc
            assert gu.ratio_full(p, out, ref) <= TOL, acc


@pytest.mark.parametrize("variant", all_variants())
def test_beta_zero_does_not_read_c(variant):
    p = inputs.make_problem(150, 260, 70, dist="normal", seed=11, beta=0.0, c_fill="nan")
    gu.say("beta=0 NaN C", g.sgemm_variant_name(variant))
    for acc, out in run_all_modes(p, variant):
        assert np.all(np.isfinite(out)), acc
        assert gu.ratio_full(p, out) <= TOL, acc


# ------------------------------------------------------------------ properties
@pytest.mark.parametrize("variant", all_variants())
def test_deterministic(variant):
    p = cached_problem("ragged_1000x1023x999")
    gu.say("determinism", g.sgemm_variant_name(variant))
    for acc in gu.allowed_accesses(p, variant=variant):
        a = gu.run(p, variant=variant, access=acc)
        b = gu.run(p, variant=variant, access=acc)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), acc


@pytest.mark.parametrize("variant", all_variants())
def test_zero_padding_invariance(variant):
    # the ragged problem inside a zero-padded larger one (same K, so the same
    # K tiles): C[:M, :N] is bit for bit the same
    p = inputs.make_problem(200, 301, 77, dist="upm1", seed=3, alpha=1.5, beta=-0.5, c_fill="upm1")
    Mb, Nb = 256, 384
    big = inputs.make_problem(Mb, Nb, 77, dist="upm1", seed=3)
    big.A.zero_(); big.B.zero_(); big.C.zero_()
    big.A[:200] = p.A
    big.B[:, :301] = p.B
    big.C[:200, :301] = p.C
    big.alpha, big.beta = p.alpha, p.beta
    gu.say("zero-padding invariance", g.sgemm_variant_name(variant))
    # N = 301 takes 32-bit accesses, or the build loading A and B 16 bytes at
    # a time at 4-byte alignment; N = 384 also the 128-bit build where the
    # variant takes it at this K (the variants reading A 128 bits at a time
    # need K % 4 == 0, so they do not here): the same arithmetic
    small = gu.run(p, variant=variant)
    large = gu.run(big, variant=variant)
    ref_mode = gu.auto_access(big, variant)
    assert gu.same_sum_order(variant, gu.auto_access(p, variant), ref_mode)
    assert np.array_equal(small.view(np.uint32), large[:200, :301].copy().view(np.uint32))
    # the access modes of one kernel family compute the same sums in the same
    # order (bit for bit); a build of the other family is held to the pass rule
    for acc in gu.allowed_accesses(big, variant=variant):
        other = gu.run(big, variant=variant, access=acc)
        if gu.same_sum_order(variant, acc, ref_mode):
            assert np.array_equal(other.view(np.uint32), large.view(np.uint32)), acc
        else:
            assert gu.ratio_full(big, other) <= TOL, acc


def test_runs_on_a_side_stream():
    p = cached_problem("square256_u01")
    s = torch.cuda.Stream()
    gu.say("side stream")
    with torch.cuda.stream(s):
        out = gu.run(p, stream=s)
    assert gu.ratio_full(p, out, cached_oracle("square256_u01")) <= TOL


@pytest.mark.parametrize("mn", [(0, 37), (29, 0), (0, 0)])
def test_empty_c_launches_nothing_and_touches_nothing(mn):
    M, N = mn
    K = 19
    p = inputs.make_problem(max(M, 1), max(N, 1), K, dist="upm1", seed=41, beta=0.5, c_fill="upm1")
    oa, _, a = gu.to_gpu(p.A)
    ob, _, b = gu.to_gpu(p.B)
    oc, _, c = gu.to_gpu(p.C)
    before = [o.cpu().numpy().copy() for o in (oa, ob, oc)]
    gu.say("empty", M, N, K)
    for v in all_variants():
        assert g.sgemm_variant(v, M, N, K, 1.0, a, K, b, max(N, 1), 0.5, c, max(N, 1)) == 0
    assert g.sgemm(M, N, K, 1.0, a, K, b, max(N, 1), 0.5, c, max(N, 1)) == 0
    torch.cuda.synchronize()
    for o, h in zip((oa, ob, oc), before):
        assert np.array_equal(o.cpu().numpy().view(np.uint32), h.view(np.uint32))


def test_device_fp32_peak_from_properties():
    cu, clk, tf = g.sgemm_device_fp32_peak(0)
    gu.say("device", cu, "CUs", clk, "kHz", tf, "TFLOP/s")
    assert cu > 0 and clk > 0
    assert tf == pytest.approx(cu * 256 * clk * 1e3 / 1e12, rel=1e-12)


# ------------------------------------------------------------------ full sizes, sampled
FULL = ["square2048_normal", "square4096_upm1", "square8192_normal", "lowk_16384x16384x128",
        "square16384_normal"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_auto_path(name):
    """The full workloads through sgemm(): whole rows {0, M-1, 62 seeded},
    whole columns {0, N-1, 62 seeded} and 4096 seeded random points against
    the oracle."""
    p = inputs.workload_problem(name)
    gu.say("full size", name, "auto variant",
           g.sgemm_variant_name(g.sgemm_select_variant(0, p.M, p.N, p.K)))
    out = gu.run(p)
    r, rows, cols = gu.ratio_lines(p, out, seed=17)
    assert len(rows) >= 60 and len(cols) >= 60 and rows[0] == 0 and rows[-1] == p.M - 1
    assert r <= TOL, (name, r)


@pytest.mark.parametrize("shape", [(8191, 8191, 8191, 1.0, 0.0), (4097, 4095, 4093, 1.5, -0.5)])
def test_full_size_sampled_odd_sizes(shape):
    """Large shapes whose rows are only 4-byte aligned (the builds loading A
    and B 16 bytes at a time at 4-byte alignment) through sgemm() and
    sgemm_ws(), sampled as the full workloads are."""
    M, N, K, alpha, beta = shape
    p = inputs.make_problem(M, N, K, dist="normal", seed=29, alpha=alpha, beta=beta,
                            c_fill="upm1" if beta != 0 else None)
    gu.say("full size odd", shape, g.sgemm_variant_name(g.sgemm_select_variant(0, M, N, K)))
    out = gu.run(p)
    r, rows, cols = gu.ratio_lines(p, out, seed=31)
    assert rows[-1] == M - 1 and cols[-1] == N - 1
    assert r <= TOL, (shape, r)
    need = g.sgemm_workspace_size(M, N, K)
    ws = torch.full((max(need, 256) // 4 + 64,), float("nan"), dtype=torch.float32, device="cuda")
    oa, _, a = gu.to_gpu(p.A)
    ob, _, b = gu.to_gpu(p.B)
    oc, first, c = gu.to_gpu(p.C)
    g.sgemm_ws(M, N, K, alpha, a, p.lda, b, p.ldb, beta, c, p.ldc, workspace=ws)
    torch.cuda.synchronize()
    out2 = oc.cpu().numpy()[first:first + p.C.numel()].reshape(p.C.shape)
    r2, _, _ = gu.ratio_lines(p, out2, seed=31)
    assert r2 <= TOL, (shape, "sgemm_ws", r2)
    del oa, ob, oc, ws


@pytest.mark.parametrize("name", ["square4096_upm1", "square8192_normal"])
def test_full_size_sampled_valu_path(name):
    p = inputs.workload_problem(name)
    gu.say("full size", name, "VALU")
    out = gu.run(p, path=g.SGEMM_PATH_VALU)
    r, _, _ = gu.ratio_lines(p, out, n_lines=30, n_random=2048, seed=19)
    assert r <= TOL


def test_huge_leading_dimension_takes_checked_accesses():
    # lda = 2.2M floats: (256 + 1) * lda * 4 bytes is past 2^31, so the
    # 256-row variant cannot use 31-bit buffer offsets and falls back to the
    # per-element checked kernel; the forced buffer modes are refused.
    M, N, K, lda = 8, 64, 64, 2_200_000
    p = inputs.make_problem(M, N, K, dist="upm1", seed=23, alpha=0.75, beta=0.5, c_fill="upm1",
                            lda=lda)
    v = [i for i in all_variants() if g.sgemm_variant_name(i) == "mfma_256x256x32_w64x64_w16_kcd"][0]
    assert g.sgemm_variant_tile(v)[1:] == (256, 256)
    gu.say("huge lda", lda, g.sgemm_variant_name(v))
    out = gu.run(p, variant=v)
    assert gu.ratio_full(p, out) <= TOL
    oa, _, a = gu.to_gpu(p.A)
    ob, _, b = gu.to_gpu(p.B)
    oc, _, c = gu.to_gpu(p.C)
    for acc in (g.SGEMM_ACCESS_BUFFER_128, g.SGEMM_ACCESS_BUFFER_32, g.SGEMM_ACCESS_BUFFER_128_AB):
        assert g.sgemm_variant_access(v, acc, M, N, K, 0.75, a, lda, b, N, 0.5, c, N,
                                      check=False) == -23
    torch.cuda.synchronize()
    del oa, ob, oc


def test_sgemm_ws_plan_beyond_31_bit_offsets_runs_whole_tiles():
    """A split plan whose 64 x 64 block cannot address A in 31 bits (lda = 9M
    floats: 65 rows span more than 2^31 bytes) runs as sgemm() does instead of
    being refused: here the 32 x 32 block, whose 33 rows still fit."""
    M, N, K, lda = 8, 64, 4096, 9_000_000
    p = inputs.make_problem(M, N, K, dist="upm1", seed=67, alpha=1.25, beta=-0.5, c_fill="upm1",
                            lda=lda)
    need = g.sgemm_workspace_size(M, N, K)
    assert need > 0 and g.sgemm_select_splits(M, N, K) > 1
    ws = torch.full((need // 4 + 64,), float("nan"), dtype=torch.float32, device="cuda")
    oa, _, a = gu.to_gpu(p.A)
    ob, _, b = gu.to_gpu(p.B)
    oc, first, c = gu.to_gpu(p.C)
    assert g.sgemm_operands_load16(a, lda, b, N, c, N)
    gu.say("sgemm_ws huge lda", lda)
    rc = g.sgemm_ws(M, N, K, p.alpha, a, lda, b, N, p.beta, c, N, workspace=ws, check=False)
    torch.cuda.synchronize()
    assert rc == 0, rc
    host = oc.cpu().numpy()
    assert np.all(np.isnan(np.concatenate([host[:first], host[first + p.C.numel():]])))
    assert gu.ratio_full(p, host[first:first + p.C.numel()].reshape(p.C.shape)) <= TOL
    del oa, ob, oc


@pytest.mark.parametrize("path", [g.SGEMM_PATH_AUTO, g.SGEMM_PATH_VALU])
def test_c_beyond_4_gib(path):
    """C of 40000 x 32768 floats (5.2 GB): byte offsets into C pass 2^32 and
    element counts pass 2^30, so any 32-bit address arithmetic would land in
    the wrong place.  Sub-blocks at the first, middle and last tile rows and
    columns are checked against the oracle on the same sub-problem."""
    M, N, K, alpha, beta, c0 = 40000, 32768, 5, 1.5, -0.5, 0.25
    p = inputs.make_problem(M, N, K, dist="upm1", seed=29, alpha=alpha, beta=beta, with_c=False)
    a, b = p.A.cuda(), p.B.cuda()
    c = torch.full((M, N), c0, dtype=torch.float32, device="cuda")
    gu.say("C beyond 4 GiB", M, N, K, "path", path)
    g.sgemm_path(path, M, N, K, alpha, a, K, b, N, beta, c, N)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = sorted(set([0, 1, 127, 128, 255, 256, M // 2, M - 257, M - 256, M - 129, M - 128, M - 2,
                       M - 1] + list(rng.integers(0, M, 24))))
    cols = sorted(set([0, 3, 4, 255, 256, N // 2, N - 257, N - 256, N - 5, N - 4, N - 1]
                      + list(rng.integers(0, N, 24))))
    ri = torch.tensor(rows, dtype=torch.long, device="cuda")
    ci = torch.tensor(cols, dtype=torch.long, device="cuda")
    got = c.index_select(0, ri).index_select(1, ci).cpu().numpy()
    del c
    torch.cuda.empty_cache()
    As = p.A[rows].contiguous().numpy().reshape(-1)
    Bs = p.B[:, cols].contiguous().numpy().reshape(-1)
    Cs = np.full(len(rows) * len(cols), c0, dtype=np.float32)
    ref, den = oracle.sgemm(len(rows), len(cols), K, alpha, As, K, Bs, len(cols), beta, Cs,
                            len(cols))
    assert oracle.max_error_ratio(got, ref, den) <= TOL


def random_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N, K = (int(x) for x in rng.integers(1, 700, 3))
        if i % 4 == 3:  # few tiles, long K: sgemm_ws splits K
            M, N = (int(x) for x in rng.integers(1, 300, 2))
            K = int(rng.integers(2048, 6000))
        alpha = float(rng.choice([1.0, -0.5, 2.0, 0.0, 1.25]))
        beta = float(rng.choice([0.0, 1.0, -0.75, 0.5]))
        pads = [int(x) for x in rng.integers(0, 6, 3)]
        offs = tuple(int(x) for x in rng.integers(0, 4, 3))
        if i % 8 == 3:  # operands that allow 128-bit accesses; the rest of the
            # long-K configurations keep odd sizes and offsets (16-byte loads at
            # 4-byte alignment)
            N, K = -(-N // 4) * 4, -(-K // 4) * 4
            pads = [4 * (x % 2) for x in pads]
            offs = (0, 0, 0)
        out.append((i, M, N, K, alpha, beta, pads, offs))
    return out


@pytest.mark.parametrize("cfg", random_configs(60, 2024), ids=lambda c: f"r{c[0]}")
def test_random_configs_every_entry_point(cfg):
    """Seeded random sizes, leading-dimension padding, base misalignment and
    alpha/beta, through sgemm, sgemm_ws (which may split K: every fourth
    configuration has few tiles and long K, half of them with 128-bit
    operands) and the VALU path."""
    i, M, N, K, alpha, beta, pads, offs = cfg
    p = inputs.make_problem(M, N, K, dist="upm1", seed=100 + i, alpha=alpha, beta=beta,
                            c_fill="upm1", lda=K + pads[0], ldb=N + pads[1], ldc=N + pads[2])
    ref_den = gu.oracle_full(p)
    gu.say("random", cfg)
    out = gu.run(p, offsets=offs)
    assert gu.ratio_full(p, out, ref_den) <= TOL
    out = gu.run(p, path=g.SGEMM_PATH_VALU, offsets=offs)
    assert gu.ratio_full(p, out, ref_den) <= TOL
    # sgemm_ws with the workspace it asks for (NaN-filled: any contents)
    need = g.sgemm_workspace_size(M, N, K)
    ws = torch.full((max(need, 256) // 4 + 64,), float("nan"), dtype=torch.float32, device="cuda")
    oa, _, a = gu.to_gpu(p.A, offs[0])
    ob, _, b = gu.to_gpu(p.B, offs[1])
    oc, first, c = gu.to_gpu(p.C, offs[2])
    if i % 4 == 3:
        assert g.sgemm_operands_load16(a, p.lda, b, p.ldb, c, p.ldc)
        assert g.sgemm_select_splits(M, N, K) > 1, (M, N, K)
    g.sgemm_ws(M, N, K, alpha, a, p.lda, b, p.ldb, beta, c, p.ldc, workspace=ws)
    torch.cuda.synchronize()
    got = oc.cpu().numpy()[first:first + p.C.numel()].reshape(p.C.shape)
    assert oracle.max_error_ratio(got[:, :N], *ref_den) <= TOL


# ------------------------------------------------------------------ split-K
def split_variants():
    return [v for v in all_variants() if g.variant_has_splitk(v)]


def run_split(p, variant, splits, ws=None):
    """One split-K launch; returns (C, workspace tensor)."""
    need = g.sgemm_splitk_workspace_size(variant, splits, p.M, p.N)
    if ws is None:  # any contents: fill with NaN to show none of it leaks through
        ws = torch.full((max(need, 256) // 4 + 64,), float("nan"), dtype=torch.float32,
                        device="cuda")
    oa, _, a = gu.to_gpu(p.A)
    ob, _, b = gu.to_gpu(p.B)
    oc, first, c = gu.to_gpu(p.C)
    g.sgemm_splitk(variant, splits, p.M, p.N, p.K, p.alpha, a, p.lda, b, p.ldb, p.beta, c, p.ldc,
                   workspace=ws)
    torch.cuda.synchronize()
    host = oc.cpu().numpy()
    n = p.C.numel()
    guard = np.concatenate([host[:first], host[first + n:]])
    assert np.all(np.isnan(guard)), "write outside C's extent"
    return host[first:first + n].reshape(p.C.shape), ws


@pytest.mark.parametrize("variant", split_variants())
@pytest.mark.parametrize("splits", [2, 3, 4, 7])
def test_splitk_matches_oracle(variant, splits):
    # the last: K % 4 != 0 and NaN in A's pad columns (lda = K + 2)
    for (M, N, K, alpha, beta, lda) in [(200, 301, 777, 1.5, -0.5, None), (256, 256, 256, 1.0, 0.0, None),
                                        (65, 130, 1030, -1.0, 1.0, None), (64, 64, 40, 2.0, 0.5, None),
                                        (70, 50, 701, 1.0, 1.0, 703)]:
        p = inputs.make_problem(M, N, K, dist="upm1", seed=M + K, alpha=alpha, beta=beta,
                                c_fill="upm1" if beta != 0 else None, lda=lda)
        gu.say("split-K", M, N, K, splits, g.sgemm_variant_name(variant))
        out, ws = run_split(p, variant, splits)
        assert gu.ratio_full(p, out) <= TOL, (M, N, K, splits)


@pytest.mark.parametrize("variant", split_variants())
def test_splitk_deterministic_and_reusable(variant):
    p = cached_problem("ragged_1000x1023x999")
    gu.say("split-K determinism", g.sgemm_variant_name(variant))
    out1, ws = run_split(p, variant, 4)
    out2, ws = run_split(p, variant, 4, ws)   # same workspace again
    assert np.array_equal(out1.view(np.uint32), out2.view(np.uint32))
    assert gu.ratio_full(p, out1, cached_oracle("ragged_1000x1023x999")) <= TOL


@pytest.mark.parametrize("variant", split_variants())
def test_splitk_closed_form_exact(variant):
    p = inputs.make_problem(192, 128, 1000, dist="ones_twos")
    gu.say("split-K closed form", g.sgemm_variant_name(variant))
    for splits in (2, 5):
        out, _ = run_split(p, variant, splits)
        assert np.all(out == 2000.0), splits


# ------------------------------------------------------------------ stream-K
def streamk_variants():
    return [v for v in all_variants() if g.variant_has_streamk(v)]


def run_streamk(p, variant, workers, ws=None):
    """One stream-K launch; returns (C, workspace tensor)."""
    need = g.sgemm_streamk_workspace_size(variant, workers)
    assert need > 0
    if ws is None:  # any contents: fill with NaN to show none of it leaks through
        ws = torch.full((need // 4 + 64,), float("nan"), dtype=torch.float32, device="cuda")
    oa, _, a = gu.to_gpu(p.A)
    ob, _, b = gu.to_gpu(p.B)
    oc, first, c = gu.to_gpu(p.C)
    g.sgemm_streamk(variant, workers, p.M, p.N, p.K, p.alpha, a, p.lda, b, p.ldb, p.beta, c, p.ldc,
                    workspace=ws)
    torch.cuda.synchronize()
    host = oc.cpu().numpy()
    n = p.C.numel()
    guard = np.concatenate([host[:first], host[first + n:]])
    assert np.all(np.isnan(guard)), "write outside C's extent"
    return host[first:first + n].reshape(p.C.shape), ws


# Shapes whose tile counts leave a remainder for the worker counts below
# (from 2 tiles of 256 x 256 to 20 of 64 x 64, so the shared tiles range from
# all of them to a few), with K from 2 K tiles (most workers hold nothing) to
# 65 (each shared tile spread over several workers).
STREAMK_SHAPES = [(200, 301, 777, 1.5, -0.5, None), (300, 260, 1030, -1.0, 1.0, None),
                  (520, 130, 96, 2.0, 0.5, None), (64, 64, 40, 1.0, 0.0, None),
                  (150, 70, 301, 1.0, 1.0, 302)]  # the last: NaN in A's pad column, K % 4 != 0


@pytest.mark.parametrize("variant", streamk_variants())
@pytest.mark.parametrize("workers", [3, 5, 16, 256])
def test_streamk_matches_oracle(variant, workers):
    for (M, N, K, alpha, beta, lda) in STREAMK_SHAPES:
        p = inputs.make_problem(M, N, K, dist="upm1", seed=M + K + 1, alpha=alpha, beta=beta,
                                c_fill="upm1" if beta != 0 else None, lda=lda)
        gu.say("stream-K", M, N, K, workers, g.sgemm_variant_name(variant))
        out, _ = run_streamk(p, variant, workers)
        assert gu.ratio_full(p, out) <= TOL, (M, N, K, workers)


@pytest.mark.parametrize("variant", streamk_variants())
def test_streamk_deterministic_reusable_and_exact(variant):
    p = cached_problem("ragged_1000x1023x999")
    gu.say("stream-K determinism", g.sgemm_variant_name(variant))
    out1, ws = run_streamk(p, variant, 7)
    out2, ws = run_streamk(p, variant, 7, ws)   # same workspace again
    assert np.array_equal(out1.view(np.uint32), out2.view(np.uint32))
    assert gu.ratio_full(p, out1, cached_oracle("ragged_1000x1023x999")) <= TOL
    q = inputs.make_problem(192, 128, 1000, dist="ones_twos")
    for workers in (3, 7):
        out, _ = run_streamk(q, variant, workers)
        assert np.all(out == 2000.0), workers


def kcd_variants():
    return [v for v in all_variants() if g.sgemm_variant_name(v).endswith("_kcd")]


@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("variant", kcd_variants())
def test_tile_order_with_ragged_tile_columns(variant, aligned):
    """11 tile columns (8 + 3) and 3 tile rows, both ragged: the blocks with
    A in K order keep each XCD on columns x, x + 8 and deal the last 3
    columns out at the end, so every tile must still be computed exactly
    once, by every build: each access mode the operands allow (aligned:
    the 128-bit build too), split-K and stream-K (whole tiles first, then
    one shared)."""
    _, bm, bn = g.sgemm_variant_tile(variant)
    M, N, K = (3 * bm - 5, 11 * bn - 8, 76) if aligned else (3 * bm - 5, 11 * bn - 7, 77)
    p = inputs.make_problem(M, N, K, dist="upm1", seed=M + N, alpha=1.25, beta=-0.5, c_fill="upm1")
    ref_den = gu.oracle_full(p)
    gu.say("ragged tile columns", M, N, K, g.sgemm_variant_name(variant))
    modes = gu.allowed_accesses(p, variant=variant)
    assert (g.SGEMM_ACCESS_BUFFER_128 in modes) == aligned
    for acc, out in run_all_modes(p, variant):
        assert gu.ratio_full(p, out, ref_den) <= TOL, gu.ACCESS_NAMES[acc]
    if g.variant_has_splitk(variant):
        out, _ = run_split(p, variant, 3)
        assert gu.ratio_full(p, out, ref_den) <= TOL, "split-K"
    if g.variant_has_streamk(variant):
        out, _ = run_streamk(p, variant, 16)  # 33 tiles: 32 whole, 1 shared
        assert gu.ratio_full(p, out, ref_den) <= TOL, "stream-K"


@pytest.mark.parametrize("name", ["5120x5120x5120", "3072x3072x3072", "13824x13824x13824",
                                  "7168x7168x7168"])
def test_sgemm_ws_streamk_full_size_sampled(name):
    """Shapes whose last round of tiles leaves slots idle: sgemm_ws shares
    the K tiles of the rest over one worker per slot (checked on sampled
    points against the oracle).  With no workspace it runs whole tiles, at
    7168^3 cut by columns into two launches and at 5120^3 into three pieces
    (whole rows and columns on both sides of each cut are checked).  At 13824^3 neither tile grid has a multiple
    of 8 columns (54 of 256 x 256, 108 of 128 x 128), so both runs take the
    per-XCD column order."""
    M, N, K = (int(x) for x in name.split("x"))
    p = inputs.make_problem(M, N, K, dist="normal", seed=37, alpha=0.75, beta=0.5, c_fill="upm1")
    workers = g.sgemm_select_streamk(M, N, K)
    assert workers > 0
    _, cut_r, cut_c, _ = g.sgemm_select_pieces(M, N, K)
    assert (cut_r > 0) == (M in (7168, 5120)), (cut_r, cut_c)
    need = g.sgemm_workspace_size(M, N, K)
    ws = torch.full((need // 4 + 64,), float("nan"), dtype=torch.float32, device="cuda")
    rows, cols = inputs.sample_points(M, N, n_random=2048, seed=41)
    if cut_r > 0:
        r1, c1 = cut_lines(M, N, cut_r, cut_c)
        rows = np.concatenate([rows, r1])
        cols = np.concatenate([cols, c1])
    for workspace in (ws, None):
        oa, _, a = gu.to_gpu(p.A)
        ob, _, b = gu.to_gpu(p.B)
        oc, first, c = gu.to_gpu(p.C)
        gu.say("sgemm_ws stream-K", name, "workers", workers, "workspace", workspace is not None)
        g.sgemm_ws(M, N, K, p.alpha, a, p.lda, b, p.ldb, p.beta, c, p.ldc, workspace=workspace)
        torch.cuda.synchronize()
        out = oc.cpu().numpy()[first:first + p.C.numel()].reshape(p.C.shape)
        assert gu.ratio_points(p, out, rows, cols) <= TOL, workspace is not None
        del oa, ob, oc


def cut_lines(M, N, rows, cols):
    """Whole rows and columns on both sides of a cut at (rows, cols), and C's
    first and last ones, as (rows, cols) point vectors."""
    er = sorted({x for x in (0, rows - 1, rows, M - 1) if 0 <= x < M})
    ec = sorted({x for x in (0, cols - 1, cols, N - 1) if 0 <= x < N})
    r = np.concatenate([np.repeat(er, N), np.tile(np.arange(M), len(ec))]).astype(np.int32)
    c = np.concatenate([np.tile(np.arange(N), len(er)), np.repeat(ec, M)]).astype(np.int32)
    return r, c


@pytest.mark.parametrize("offsets", [(0, 0, 0), (1, 2, 3)])
@pytest.mark.parametrize("beta", [0.0, -0.75])
@pytest.mark.parametrize("shape", [(8256, 2047, 2048, 8192, 2047, 15), (4300, 4301, 2048, 4096, 4096, 15),
                                   (2946, 2901, 2048, 2944, 2816, 12), (4122, 2098, 1536, 4096, 2048, 10)])
def test_pieces_through_sgemm(shape, offsets, beta):
    """Shapes that sgemm() cuts into pieces: 8256 x 2047 x 2048 by rows (the
    first 8192 rows on 256 x 256 tiles, the last 64 with their own block),
    4300 x 4301 x 2048 in three (4096 x 4096 on 256 x 256 tiles, the 205
    columns right of it over those rows, the 204 rows below over every
    column), 2946 x 2901 x 2048 in three with the first piece on 128 x 128
    tiles (2944 x 2816; then 85 columns, then 2 rows), 4122 x 2098 x 1536 with
    it on 128 x 256 tiles (4096 x 2048; then 50 columns, then 26 rows).  N % 4 != 0 and the misaligned bases take the builds loading A
    and B 16 bytes at a time at 4-byte alignment; ldc is padded (its pad
    columns must keep their bits) and nothing outside C is written.  beta = 0
    runs over a NaN C, so every element must come out finite: each is written
    by a piece.  Whole rows and columns on both sides of each cut, C's edges
    and random points against the oracle."""
    M, N, K, rows, cols, first = shape
    assert g.sgemm_select_pieces(M, N, K) == (0, rows, cols, first)
    p = inputs.make_problem(M, N, K, dist="upm1", seed=47, alpha=1.25, beta=beta,
                            c_fill="upm1" if beta != 0 else "nan", lda=K + 3, ldb=N + 1, ldc=N + 5)
    gu.say("pieces via sgemm", M, N, K, "cut", rows, cols, "beta", beta, "offsets", offsets)
    out = gu.run(p, offsets=offsets)
    assert gu.pad_untouched(p, out)
    assert np.all(np.isfinite(out[:, :N]))
    r1, c1 = cut_lines(M, N, rows, cols)
    r2, c2 = inputs.sample_points(M, N, n_random=4096, seed=43)
    assert gu.ratio_points(p, out, np.concatenate([r1, r2]), np.concatenate([c1, c2])) <= TOL


@pytest.mark.parametrize("name", ["square256_u01", "ragged_1000x1023x999", "512x512x8192",
                                  "1024x1024x4096"])
def test_sgemm_ws_auto(name):
    if name[0].isdigit():
        M, N, K = (int(x) for x in name.split("x"))
        p = inputs.make_problem(M, N, K, dist="normal", seed=31, alpha=0.5, beta=-1.0, c_fill="u01")
        ref_den = gu.oracle_full(p)
    else:
        p = cached_problem(name)
        ref_den = cached_oracle(name)
    need = g.sgemm_workspace_size(p.M, p.N, p.K)
    ws = torch.zeros(max(need, 256) // 4 + 64, dtype=torch.float32, device="cuda")
    oa, _, a = gu.to_gpu(p.A)
    ob, _, b = gu.to_gpu(p.B)
    oc, first, c = gu.to_gpu(p.C)
    gu.say("sgemm_ws", name, "splits", g.sgemm_select_splits(p.M, p.N, p.K), "bytes", need)
    g.sgemm_ws(p.M, p.N, p.K, p.alpha, a, p.lda, b, p.ldb, p.beta, c, p.ldc, workspace=ws)
    torch.cuda.synchronize()
    out = oc.cpu().numpy()[first:first + p.C.numel()].reshape(p.C.shape)
    assert gu.ratio_full(p, out, ref_den) <= TOL
    # too small a workspace falls back to the unsplit kernel
    oc2, first2, c2 = gu.to_gpu(p.C)
    g.sgemm_ws(p.M, p.N, p.K, p.alpha, a, p.lda, b, p.ldb, p.beta, c2, p.ldc, workspace=ws,
               workspace_bytes=64)
    torch.cuda.synchronize()
    out2 = oc2.cpu().numpy()[first2:first2 + p.C.numel()].reshape(p.C.shape)
    assert gu.ratio_full(p, out2, ref_den) <= TOL
