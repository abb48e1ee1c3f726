"""Host logic of bench.py that needs no GPU: the parity check beside the CPU
baseline, and the shape of its report."""
import importlib.util
import os
import sys

import numpy as np
import pytest

from fp32_gemm_03_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        spec.loader.exec_module(mod)
    finally:
        sys.argv = argv
    return mod


@pytest.mark.parametrize("beta", [0.0, -0.5])
def test_parity_of_the_first_rows_against_the_oracle(bench, beta):
    p = inputs.make_problem(300, 260, 129, dist="upm1", seed=2, alpha=1.5, beta=beta,
                            c_fill="upm1" if beta else None)
    # float32 rounding of the exact result: well inside the pass rule
    exact = p.alpha * (p.A.double() @ p.B.double()) + p.beta * p.C.double()
    rows = exact.float().double().numpy()[:200]
    base, parity = bench.cpu_baseline(p, target_s=0.05, gpu_rows=rows)
    assert base["kind"] == "oracle" and base["cores"] >= 1 and base["value"] > 0
    assert parity["pass"] and parity["max_err_ratio"] <= bench.TOLERANCE
    assert 0 < parity["rows"] <= 200 and parity["elements"] == parity["rows"] * p.N
    # one element off by 1e-3 (its denominator is at most about 1.5 * 129) fails the rule
    bad = rows.copy()
    bad[3, 7] += 1e-3
    assert not bench.cpu_baseline(p, target_s=0.05, gpu_rows=bad)[1]["pass"]
    # a NaN anywhere fails too
    bad = rows.copy()
    bad[0, 0] = np.nan
    assert not bench.cpu_baseline(p, target_s=0.05, gpu_rows=bad)[1]["pass"]


def test_no_parity_without_gpu_rows(bench):
    p = inputs.make_problem(64, 64, 64, dist="u01", seed=0)
    base, parity = bench.cpu_baseline(p, target_s=0.01)
    assert parity is None and base["unit"] == "TFLOP/s"


def test_whole_problem_oracle_and_parity(bench):
    """The secondary workloads' check: the oracle on the whole problem, every
    element of C against it, the sample labelled as the whole problem."""
    p = inputs.make_problem(120, 77, 45, dist="upm1", seed=5, alpha=-0.5, beta=1.5, c_fill="upm1")
    exact = p.alpha * (p.A.double() @ p.B.double()) + p.beta * p.C.double()
    c = exact.float().double().numpy()
    base, parity = bench.cpu_baseline(p, gpu_rows=c, full=True)
    assert base["sample"].startswith("the whole 120x77x45 problem")
    assert parity["rows"] == 120 and parity["elements"] == 120 * 77 and parity["pass"]
    assert parity["against"].startswith("every element")
    bad = c.copy()
    bad[119, 76] += 1e-2
    assert not bench.cpu_baseline(p, gpu_rows=bad, full=True)[1]["pass"]
    # every secondary workload but the band-only ones runs the whole oracle
    assert set(bench.BAND_ONLY) <= set(bench.SECONDARY)
