"""Plant mistakes in the CPU reference (on the CPU, in temporary builds) and
check that its pins catch every one of them.

Each mutant is oracle_sgemm.c with one plausible slip: a dropped term, a
wrong sign, a transposed or mis-strided operand, a missing BLAS convention,
a precision loss.  A mutant that passed every pin would mean the pins could
not tell that slip from the real thing.
"""

import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build
from oracle import oracle
from tests import oracle_pins

MUTANTS = {
    "drop_last_k": ("for (int64_t k = 0; k < jb->K; ++k)", "for (int64_t k = 0; k + 1 < jb->K; ++k)"),
    "drop_first_k": ("for (int64_t k = 0; k < jb->K; ++k)", "for (int64_t k = 1; k < jb->K; ++k)"),
    "drop_last_col": ("for (int64_t j = 0; j < jb->N; ++j) {\n                    const double p",
                      "for (int64_t j = 0; j + 1 < jb->N; ++j) {\n                    const double p"),
    "sign_of_product": ("acc[j] += p;", "acc[j] -= p;"),
    "sign_of_beta": ("out += jb->beta *", "out -= jb->beta *"),
    "alpha_dropped": ("jb->alpha * acc[j]", "acc[j]"),
    "a_transposed": ("jb->A[i * jb->lda + k]", "jb->A[k * jb->lda + i]"),
    "b_transposed": ("(double)brow[j]", "(double)jb->B[j * jb->ldb + k]"),
    "lda_as_k": ("jb->A[i * jb->lda + k]", "jb->A[i * jb->K + k]"),
    "ldb_as_n": ("jb->B + k * jb->ldb", "jb->B + k * jb->N"),
    "ldc_as_n": ("jb->C[i * jb->ldc + j]", "jb->C[i * jb->N + j]"),
    "c_read_when_beta_zero": ("if (jb->beta != 0.0)", "if (1)"),
    "no_alpha_zero_quick_return": ("(alpha != 0.0f) && (K > 0)", "(K > 0)"),
    "float32_products": ("const double p = a * (double)brow[j];", "const double p = (float)(a * (double)brow[j]);"),
    "float32_sum": ("acc[j] += p;", "acc[j] = (float)(acc[j] + p);"),
    "sumabs_signed": ("sab[j] += fabs(p);", "sab[j] += p;"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle_build.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, "-o", str(lib), str(path), "-lm"], check=True)
    return str(lib)


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Runs every pin against one build in a child process, so a mutant that reads
# out of bounds (a NULL C, a transposed index) cannot take the test run down;
# a crash counts as caught.
_CHILD = """
import sys
sys.path.insert(0, {root!r})
from oracle import oracle
from tests import oracle_pins
lib = oracle.load({lib!r})
caught = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lambda *a, **k: oracle.oracle_sgemm(*a, lib=lib, **k))
    except (AssertionError, ValueError):
        caught.append(pin.__name__)
print("CAUGHT", ",".join(caught))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    proc = subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT, lib=lib)],
                          capture_output=True, text=True, timeout=300)
    if proc.returncode != 0:
        return  # the mutant crashed on a pin's input: caught
    line = [ln for ln in proc.stdout.splitlines() if ln.startswith("CAUGHT")][-1]
    assert line.split(" ", 1)[1:] != [""], f"mutant {name} passed every pin"


def test_unmutated_source_passes(tmp_path):
    lib = oracle.load(_build_mutant(tmp_path, "identity", "acc[j] += p;", "acc[j] += p;"))
    for pin in oracle_pins.ALL_PINS:
        pin(lambda *a, **k: oracle.oracle_sgemm(*a, lib=lib, **k))


# Mistakes planted in the checker (oracle.py's normalised_error, a Python
# function): each variant is the function's source with one slip, compiled
# into a scratch namespace; at least one checker pin must reject it.
CHECKER_MUTANTS = {
    "strict_alpha_sign_kept": ("abs(alpha) if strict", "alpha if strict"),
    "strict_ignored": ("abs(alpha) if strict else 1.0", "1.0"),
    "beta_term_dropped": ("den = den + np.abs(beta * np.asarray(C_in, dtype=np.float64))", "pass"),
    "beta_term_always": ("if beta != 0.0:\n        den = den +", "if True:\n        den = den +"),
    "zero_den_not_checked": ("if np.any(out[zero] != 0.0):", "if False:"),
    "nan_not_checked": ("if not np.all(np.isfinite(out[np.isfinite(ref)])):", "if False:"),
}


def _checker_variant(old, new):
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(oracle.normalised_error))
    assert src.count(old) == 1, old
    ns = dict(oracle.__dict__)
    exec(compile(src.replace(old, new), "<checker mutant>", "exec"), ns)
    return ns["normalised_error"]


@pytest.mark.parametrize("name", sorted(CHECKER_MUTANTS))
def test_checker_pins_catch_mutant(name):
    fn = _checker_variant(*CHECKER_MUTANTS[name])
    caught = []
    for pin in oracle_pins.CHECKER_PINS:
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"checker mutant {name} passed every checker pin"


def test_checker_unmutated_passes():
    fn = _checker_variant("abs(alpha)", "abs(alpha)")
    for pin in oracle_pins.CHECKER_PINS:
        pin(fn)
