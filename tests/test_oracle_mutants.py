"""The oracle's pins reject plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign, a wrong scale, a transposed operand, a wrong row index),
builds it on the CPU and runs the pin suite against it: at least one pin must
fail for every mutant, and the unmodified source must pass them all.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "plora_oracle.c")

MUTANTS = {
    "scale_alpha_not_alpha_over_r": ("const double s = alphas[i] / (double)r;", "const double s = alphas[i];"),
    "branch_sign": ("Y[t * d_out + c] += s * row[c];", "Y[t * d_out + c] -= s * row[c];"),
    "dx_branch_dropped": ("dX[t * d_in + k] += s * row[k];", "dX[t * d_in + k] += 0.0 * row[k];"),
    "frozen_weight_transposed": ("acc += x[k] * w[k];\n                Y[t * d_out + c] = acc;",
                                 "acc += x[k] * W[k * d_out + c];\n                Y[t * d_out + c] = acc;"),
    "db_wrong_rows": ("const double* dy = dY + (o0 + u) * d_out;", "const double* dy = dY + u * d_out;"),
    "da_uses_h": ("const double g = Gi[u * r + j];", "const double g = (Hi ? Hi : Gi)[u * r + j];"),
    "da_scale_missing": ("dAi[(int64_t)j * d_in + k] *= s;", "dAi[(int64_t)j * d_in + k] *= 1.0;"),
    "g_uses_b_transposed": ("if (need_g) down_proj(dY + t * d_out, Bi, r, d_out, Gi + u * r);",
                            "if (need_g) down_proj(dY + t * d_out, Bi + 1, r, d_out - 1, Gi + u * r);"),
}

PIN_TESTS = [
    lambda: pins.test_hand_example_exact(),
    lambda: pins.test_b_zero_gives_frozen_output_exactly(),
    lambda: pins.test_frozen_path_matches_numpy(),
    lambda: pins.test_merge_identity(3),
    lambda: pins.test_block_diagonal_dense_form(),
    lambda: pins.test_rank1_closed_form(True),
    lambda: pins.test_finite_differences(),
]


def _failures():
    n = 0
    for f in PIN_TESTS:
        try:
            f()
        except (AssertionError, oracle.OracleError):
            n += 1
    return n


def _build(tmp_path, name, src_text):
    c = tmp_path / (name + ".c")
    so = tmp_path / (name + ".so")
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(c), "-o", str(so), "-lm"], check=True)
    return str(so)


def test_unmodified_source_passes(tmp_path):
    so = _build(tmp_path, "orig", open(SRC).read())
    with oracle.use_library(so):
        assert _failures() == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site not found: " + name
    so = _build(tmp_path, name, text.replace(old, new))
    with oracle.use_library(so):
        assert _failures() >= 1, name
