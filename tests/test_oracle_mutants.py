"""The oracle's pins catch plausible mistakes.

Each case copies ``oracle/oracle_sgemm.c``, plants one mistake in the copy (a
dropped term, a wrong sign, a transposed operand, a wrong leading dimension, a
missing scale), compiles it with gcc into a temporary directory and checks that
at least one pin of ``oracle_pins`` rejects it.  The pins run against the
mutant in a child process, so a mutant that crashes (say, by reading C when
it must not) cannot take the test run with it; a crash is reported as such and
does not count as a rejection.  The oracle itself is never modified.  CPU only.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle
from tests import oracle_pins as pins

MUTANTS = {
    # row entry (i-k-j walk)
    "rows_drop_last_k": ("for (int k = 0; k < nk; ++k) {", "for (int k = 0; k + 1 < nk; ++k) {"),
    "rows_product_at_alpha_zero": ("const int nk = b->alpha != 0.0 ? b->K : 0;", "const int nk = b->K;"),
    "rows_beta_sign": ("r += b->beta * c;", "r -= b->beta * c;"),
    "rows_transposed_B": ("const double p = a * (double)brow[j];",
                          "const double p = a * (double)b->B[(size_t)j * b->ldb + k];"),
    "rows_lda_is_K": ("b->A[(size_t)i * b->lda + k]", "b->A[(size_t)i * b->K + k]"),
    "rows_no_alpha": ("double r = b->alpha * sum[j];", "double r = sum[j];"),
    "rows_alpha_twice": ("double r = b->alpha * sum[j];", "double r = b->alpha * b->alpha * sum[j];"),
    "rows_den_drops_beta": ("d += fabs(b->beta) * fabs(c);", "(void)c;"),
    "rows_den_signed": ("abs_sum[j] += fabs(p);", "abs_sum[j] += p;"),
    "rows_reads_C_when_beta_zero": ("if (b->beta != 0.0) {", "if (1) {"),
    "rows_float_accumulator": ("sum[j] += p;", "sum[j] = (float)(sum[j] + p);"),
    # point entry (one dot product per element)
    "points_transposed_B": ("(double)B[(size_t)k * ldb + j]", "(double)B[(size_t)j * ldb + k]"),
    "points_skip_first_k": ("for (int k = 0; k < kend; ++k) {", "for (int k = 1; k < kend; ++k) {"),
    "points_product_at_alpha_zero": ("const int kend = alpha != 0.0f ? K : 0;", "const int kend = K;"),
    "points_beta_uses_alpha": ("r += (double)beta * c;", "r += (double)alpha * c;"),
    "points_ldc_is_N": ("(double)C[(size_t)i * ldc + j]", "(double)C[(size_t)i * N + j]"),
}


def _src():
    with open(oracle.SOURCE, encoding="utf-8") as f:
        return f.read()


_RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins as pins
lib = oracle.OracleLib({lib!r})
failed = []
for name, pin in pins.QUICK_PINS:
    try:
        pin(lib)
    except AssertionError:
        failed.append(name)
print("FAILED_PINS=" + ",".join(failed))
"""

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_pins(libpath):
    proc = subprocess.run([sys.executable, "-c", _RUNNER.format(root=ROOT, lib=libpath)],
                          capture_output=True, text=True, timeout=300)
    for line in proc.stdout.splitlines():
        if line.startswith("FAILED_PINS="):
            return proc.returncode, [x for x in line.split("=", 1)[1].split(",") if x]
    return proc.returncode, None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    text = _src()
    assert text.count(old) == 1, f"mutation site for {name} not unique in the oracle source"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new), encoding="utf-8")
    libpath = oracle.compile_c(str(src), str(tmp_path / "libmutant.so"))
    rc, failed = _run_pins(libpath)
    assert failed is not None, f"mutant {name} crashed the pin run (exit {rc}) instead of failing a pin"
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes_quick_pins():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "copy.c")
        with open(src, "w", encoding="utf-8") as f:
            f.write(_src())
        rc, failed = _run_pins(oracle.compile_c(src, os.path.join(d, "libcopy.so")))
        assert rc == 0 and failed == [], (rc, failed)
