"""The oracle's pins have teeth: deliberately broken copies of the oracle fail them.

Each case copies the oracle's sources to a temporary directory, plants one plausible
mistake by a text substitution in the copy, compiles it with gcc, routes the oracle
wrapper to the broken build and runs the pins. At least one pin must fail for every
mutant. Everything runs on the CPU; the real oracle is never modified.
"""

import os
import shutil

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = {
    "gate order f<->g": ("REAL fg = NAME(sigmoid)(a[hidden + j]);\n                REAL gg = TANHR(a[2 * hidden + j]);",
                         "REAL fg = NAME(sigmoid)(a[2 * hidden + j]);\n                REAL gg = TANHR(a[hidden + j]);"),
    "dropped forget term": ("c[j] = fg * c[j] + ig * gg;", "c[j] = ig * gg;"),
    "reverse runs forward": ("const int t = (d == 0) ? s : steps - 1 - s;", "const int t = s;"),
    "dropped recurrent bias": ("(REAL)b[((size_t)d * 2 + 1) * gates + r];", "(REAL)0;"),
    "no tanh on cell output": ("h[j] = og * TANHR(c[j]);", "h[j] = og * c[j];"),
    "wrong sigmoid branch": ("return e / ((REAL)1 + e);", "return (REAL)1 / ((REAL)1 + e);"),
    "reverse written to forward columns": ("y[(size_t)t * 2 * hidden + (size_t)d * hidden + j] = h[j];",
                                           "y[(size_t)t * 2 * hidden + j] = h[j];"),
    "state carried into the reverse pass": ("for (int j = 0; j < hidden; ++j) {\n            h[j] = (REAL)0;",
                                            "for (int j = 0; j < hidden && d == 0; ++j) {\n            h[j] = (REAL)0;"),
    "input projection transposed": ("acc += (REAL)wrow[k] * xv;",
                                    "acc += (REAL)w[((size_t)d * gates + (k % gates)) * in + (r % in)] * xv;"),
    "heads: ReLU instead of LeakyReLU": ("return v >= (REAL)0 ? v : slope * v;", "return v >= (REAL)0 ? v : (REAL)0;"),
    "heads: no LeakyReLU after linear1": ("h1[n] = NAME(leaky)(acc, s);", "h1[n] = acc;"),
    "heads: linear1 weight transposed": ("acc += h0[k] * (REAL)w1[(size_t)k * mid1 + n];",
                                         "acc += h0[k] * (REAL)w1[(size_t)n * mid0 + k];"),
    "heads: dropped classifier bias": ("REAL acc = (REAL)b2[c];", "REAL acc = (REAL)0;"),
    "heads: softmax instead of log-softmax": ("out[(size_t)m * classes + c] = z[c] - lse;",
                                              "out[(size_t)m * classes + c] = EXPR(z[c] - lse);"),
}


def _pins_all_pass(lib_fixture) -> bool:
    checks = [
        lambda: pins.test_one_unit_first_step_closed_form(lib_fixture),
        lambda: pins.test_one_unit_all_steps_match_torch(lib_fixture),
        lambda: pins.test_matches_torch_float64_small(lib_fixture, 3, 5, 2, 7, 2),
        lambda: pins.test_zero_recurrent_weights_scan_closed_form(lib_fixture),
        lambda: pins.test_time_reversal_symmetry(lib_fixture, 5, 3, 1, 11),
        lambda: pins.test_projection_matches_numpy_matmul(lib_fixture),
        lambda: pins.test_heads_one_unit_closed_form(lib_fixture),
        lambda: pins.test_heads_match_torch_float64(lib_fixture, 64, (16, 8, 12, 7)),
        lambda: pins.test_heads_log_softmax_normalised_and_shift_invariant(lib_fixture),
    ]
    for check in checks:
        try:
            check()
        except (AssertionError, RuntimeError):
            return False
    return True


def test_unmodified_copy_passes(tmp_path):
    src = tmp_path / "src"
    shutil.copytree(os.path.dirname(oracle.__file__), src,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    lib = oracle.compile_library(str(src / "bilstm_oracle.c"), str(tmp_path / "copy.so"))
    oracle.use_library(lib)
    try:
        assert _pins_all_pass(oracle)
    finally:
        oracle.use_library(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(tmp_path, name):
    old, new = MUTANTS[name]
    src = tmp_path / "src"
    shutil.copytree(os.path.dirname(oracle.__file__), src,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    body = (src / "lstm_body.inc").read_text()
    assert body.count(old) == 1, f"mutation anchor for {name!r} not found exactly once"
    (src / "lstm_body.inc").write_text(body.replace(old, new))
    lib = oracle.compile_library(str(src / "bilstm_oracle.c"), str(tmp_path / "mutant.so"))
    oracle.use_library(lib)
    try:
        assert not _pins_all_pass(oracle), f"mutant {name!r} passed every pin"
    finally:
        oracle.use_library(None)
