"""Plant plausible mistakes in copies of the oracle (CPU only) and check the pins catch each.

This shows that the pins in oracle_pins.py are not vacuous: a dropped term, a
wrong sign, a transposed operand, a wrong stride or a broken decoder each make
at least one pin fail.  The mutants are built in a temporary directory and run
in a child process (an out-of-bounds mutant may crash, which also counts as
caught); the real oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

import oracle

pytestmark = pytest.mark.spawns

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "drop_last_k": [("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k < K - 1; ++k)")],
    "transpose_B": [("elem(Bb, dtype, k * ldb + j)", "elem(Bb, dtype, j * ldb + k)"),
                    ("elem(Bb, dtype, k * ldb + pj[p])", "elem(Bb, dtype, pj[p] * ldb + k)")],
    "wrong_sign": [("s[j] += a * bv;", "s[j] -= a * bv;"), ("s += a * bv;", "s -= a * bv;")],
    "drop_beta": [("if (beta != 0.0) c += beta *", "if (0) c += beta *")],
    "beta_always_read": [("if (beta != 0.0) c += beta *", "if (1) c += beta *")],
    "lda_as_K": [("i * lda + k", "i * K + k"), ("pi[p] * lda + k", "pi[p] * K + k")],
    "ignore_alpha": [("double c = alpha * s[j];", "double c = s[j];"), ("double c = alpha * s;", "double c = s;")],
    "bf16_shift": [("((uint32_t)h) << 16", "((uint32_t)h) << 15")],
    "f16_bias": [("expo - 25", "expo - 24")],
    "f16_subnormal": [("ldexp((double)frac, -24)", "ldexp((double)frac, -25)")],
    "batch_stride_A": [("(size_t)(b * sA)", "(size_t)(b * sB)"), ("(size_t)(pb[p] * sA)", "(size_t)(pb[p] * sB)")],
    "c0_ldc": [("C0[b * sC + i * ldc + j]", "C0[b * sC + i * N + j]"),
               ("C0[pb[p] * sC + pi[p] * ldc + pj[p]]", "C0[pb[p] * sC + pi[p] * N + pj[p]]")],
    "tail_bias_swapped": [("bias[b * bias_stride + j];\n    if (bias_mode == 2) x += (double)bias[b * bias_stride + i]",
                           "bias[b * bias_stride + i];\n    if (bias_mode == 2) x += (double)bias[b * bias_stride + j]")],
    "tail_bias_sign": [("if (bias_mode == 1) x += ", "if (bias_mode == 1) x -= ")],
    "tail_bias_no_stride": [("bias[b * bias_stride + j]", "bias[j]")],
    "tail_residual_inside": [("double y = oracle_activation(x, act);\n    if (beta != 0.0) y += beta * (double)C0[b * sC + ldc * i + j];",
                              "if (beta != 0.0) x += beta * (double)C0[b * sC + ldc * i + j];\n    double y = oracle_activation(x, act);")],
    "tail_c0_ldc": [("C0[b * sC + ldc * i + j]", "C0[b * sC + (ldc - 1) * i + j]")],
    "tail_gelu_no_sqrt2": [("erf(x / sqrt(2.0))", "erf(x)")],
    "tail_gelu_tanh_form": [("x * 0.5 * (1.0 + erf(x / sqrt(2.0)))",
                             "x * 0.5 * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)))")],
    "tail_relu_leaky": [("x < 0.0 ? 0.0 : x", "x < 0.0 ? 0.01 * x : x")],
    "absden_signed": [("t[j] += fabs(a) * fabs(bv);", "t[j] += a * bv;"), ("t += fabs(a) * fabs(bv);", "t += a * bv;")],
}

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
lib = oracle.OracleLibrary({lib!r})
caught = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except (AssertionError, ValueError) as e:
        caught.append(pin.__name__)
print("CAUGHT", ",".join(caught))
"""


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(oracle.SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor missing: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = oracle.compile_library(str(path), str(tmp_path / f"lib_{name}.so"))
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=lib)],
                       capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return  # crashed (e.g. read out of bounds): caught
    line = [l for l in r.stdout.splitlines() if l.startswith("CAUGHT")][-1]
    assert line.split(" ", 1)[1:] and line.split(" ", 1)[1].strip(), f"no pin caught mutant {name}"
