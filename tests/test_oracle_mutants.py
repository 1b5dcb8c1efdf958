"""The oracle's pins catch plausible mistakes.

Each case copies gla_oracle.c, plants one mistake (a dropped term, a wrong sign,
index or operand), compiles the copy with gcc and runs a battery of the pins
from test_oracle.py against it.  Every mutant must fail at least one pin, and
the unmodified source must pass them all.  CPU only.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import tests.test_oracle as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "gla_oracle.c")

MUTANTS = {
    "no_decay": ("for (int64_t j = 0; j < nj; ++j) row[j] *= a;",
                 "for (int64_t j = 0; j < nj; ++j) row[j] *= 1.0;"),
    "vector_gate_scaled": ("if (J->vec) return exp(J->g[", "if (J->vec) return exp(0.5 * J->g["),
    "scalar_gate_sign": ("return exp(J->g[(b * J->T + t) * J->H + h]);",
                         "return exp(-J->g[(b * J->T + t) * J->H + h]);"),
    "no_reset_forward": ("const int reset = is_reset(J, b, t);", "const int reset = 0;"),
    "state_grad_wrong_operand": ("dS[c * nj + j] += qt[c] * dot[j];",
                                 "dS[c * nj + j] += kt[c] * dot[j];"),
    "dq_from_previous_state": ("aq += St[c * nj + j] * dot[j];", "aq += Sp[c * nj + j] * dot[j];"),
    "dg_from_current_state": ("r += dS[c * nj + j] * Sp[c * nj + j];",
                              "r += dS[c * nj + j] * St[c * nj + j];"),
    "dg_missing_alpha": ("if (J->vec) dgt[c] = a * r;", "if (J->vec) dgt[c] = r;"),
    "no_reset_backward": ("if (is_reset(J, b, t)) {\n                for (int64_t i = 0; i < gw",
                          "if (0) {\n                for (int64_t i = 0; i < gw"),
    "dk_transposed_state": ("ak += dS[c * nj + j] * vt[j];", "ak += dS[j * nj + c] * vt[j];"),
    "wrong_head_group_bwd": ("const int64_t G = H / J->Hqk, hq = h / G;\n    const int64_t nspan",
                             "const int64_t G = H / J->Hqk, hq = h % J->Hqk;\n    const int64_t nspan"),
    "no_dh0_decay": ("for (int64_t j = 0; j < nj; ++j) dS[c * nj + j] *= a;",
                     "for (int64_t j = 0; j < nj; ++j) dS[c * nj + j] *= (t > 0 ? a : 1.0);"),
}


def battery():
    """Run pins; return the names of those that fail."""
    failed = []
    checks = [
        ("hand", lambda: P.test_hand_worked_example()),
        ("brute_s", lambda: P.test_forward_matches_quadratic_form("scalar", [3, 1, 5, 2], 1)),
        ("brute_v", lambda: P.test_forward_matches_quadratic_form("vector", [3, 1, 5, 2], 2)),
        ("alpha1", lambda: P.test_alpha_one_closed_form_and_gradients()),
        ("fd_s", lambda: P.test_backward_matches_finite_differences("scalar", 1, [4, 1, 3])),
        ("fd_v", lambda: P.test_backward_matches_finite_differences("vector", 2, [1, 1, 6])),
        ("ident", lambda: P.test_gate_gradient_suffix_sum_identity("vector", [5, 1, 7, 3])),
        ("reverse", lambda: P.test_backward_is_forward_in_reverse()),
        ("gqa", lambda: P.test_head_sharing_equals_repeat_and_sum()),
    ]
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def _build_variant(tmp_path, name, src_text):
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-pthread", str(c), "-o",
                    str(so), "-lm"], check=True)
    return str(so)


def test_unmodified_source_passes_battery(tmp_path):
    src = open(SRC).read()
    so = _build_variant(tmp_path, "orig", src)
    try:
        oracle.use_library(so)
        assert battery() == []
    finally:
        oracle.use_library(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, "mutation site not found: " + name
    so = _build_variant(tmp_path, name, src.replace(old, new))
    try:
        oracle.use_library(so)
        with np.errstate(all="ignore"):
            failed = battery()
    finally:
        oracle.use_library(None)
    assert failed, "no pin caught mutant " + name
