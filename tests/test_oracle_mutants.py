"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (on the CPU, in a temporary
directory), builds it, and runs the pin suite against it; the suite must fail.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (description, text in oracle.c, replacement)
MUTANTS = [
    ("A block scale dropped", "a *= dec_e8m0(p->sfa", "a *= 1.0 + 0.0 * dec_e8m0(p->sfa"),
    ("block index off by one", "p->sfa[i * p->ld_sfa + q / p->block]",
     "p->sfa[i * p->ld_sfa + (q + 1) / p->block]"),
    ("SFB indexed by the wrong axis", "p->sfb[j * p->ld_sfb + q / p->block]",
     "p->sfb[(j + q) % 2 * p->ld_sfb + q / p->block]"),
    ("opA storage transposed", "p->op_a == 0 ? i + q * p->lda : q + i * p->lda",
     "p->op_a == 0 ? q + i * p->lda : i + q * p->lda"),
    ("opB storage transposed", "p->op_b == 0 ? q + j * p->ldb : j + q * p->ldb",
     "p->op_b == 0 ? j + q * p->ldb : q + j * p->ldb"),
    ("beta term sign", "t += p->beta * load_real", "t -= p->beta * load_real"),
    ("bias dropped", "t += load_real(p->bias, p->type_bias, i);",
     "t += 0.0 * load_real(p->bias, p->type_bias, i);"),
    ("nibble order swapped", "(idx & 1) ? (byte >> 4) : (byte & 0xf)",
     "(idx & 1) ? (byte & 0xf) : (byte >> 4)"),
    ("e4m3 exponent bias", "ldexp((double)(8 + f), e - 10)", "ldexp((double)(8 + f), e - 9)"),
    ("bf16 subnormal scale", "ldexp((double)f, -133)", "ldexp((double)f, -132)"),
    ("f16 mantissa width", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    ("gelu argument", "erf(t / sqrt(2.0))", "erf(t / 2.0)"),
    ("relu keeps negatives", "t > 0.0 ? t : 0.0", "t > 0.0 ? t : -t"),
    ("integer beta dropped", "t += (int64_t)p->beta *", "t += (int64_t)0 *"),
    ("per-tensor scale dropped", "p->a_scale * p->b_scale * acc", "p->a_scale * acc"),
    ("alpha dropped", "double t = p->alpha * (", "double t = 1.0 * ("),
    ("last k dropped", "for (int64_t q = 0; q < p->k; ++q) {", "for (int64_t q = 0; q + 1 < p->k; ++q) {"),
    ("e2m1 subnormal", "mag = 0.5 * f;", "mag = 1.0 * f;"),
    ("e5m2 exponent bias", "ldexp((double)(4 + f), e - 17)", "ldexp((double)(4 + f), e - 16)"),
    ("e5m2 top exponent taken as finite", "if (e == 31)\n        mag = f == 0 ? INFINITY : NAN;",
     "if (e == 32)\n        mag = f == 0 ? INFINITY : NAN;"),
    ("e5m2 subnormal scale", "ldexp((double)f, -16); /* f/4 * 2^-14 */", "ldexp((double)f, -14); /* f/4 * 2^-14 */"),
    ("integer relu keeps negatives, zeroes positives", "if (p->act == ORC_ACT_RELU && t < 0)",
     "if (p->act == ORC_ACT_RELU && t > 0)"),
    ("gelu by the tanh approximation", "return 0.5 * t * (1.0 + erf(t / sqrt(2.0))); /* erf form of GELU */",
     "return 0.5 * t * (1.0 + tanh(sqrt(2.0 / 3.141592653589793) * (t + 0.044715 * t * t * t)));"),
    ("gelu without the factor one half", "return 0.5 * t * (1.0 + erf(t / sqrt(2.0))); /* erf form of GELU */",
     "return t * (1.0 + erf(t / sqrt(2.0)));"),
    ("MX output: E2M1's largest exponent off by one", "emax = 2; ncodes = 8;", "emax = 1; ncodes = 8;"),
    ("MX output: ties to the odd code", "(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    ("MX output: large magnitudes not clamped", "for (int c = 0; c < ncodes && a < top; ++c)",
     "for (int c = 0; c < ncodes; ++c)"),
    ("MX output: scale bias", "*scale = (uint8_t)(x + 127);", "*scale = (uint8_t)(x + 126);"),
    ("MX output: element sign dropped", "codes[t] = (uint8_t)(best | (signbit(vals[t]) ? (1 << sign_bit) : 0));",
     "codes[t] = (uint8_t)best;"),
    ("MX output: E5M2 clamps one code short", "emax = 15; ncodes = 124;", "emax = 15; ncodes = 123;"),
    ("e2m3 exponent bias", "ldexp((double)(8 + f), e - 4)", "ldexp((double)(8 + f), e - 3)"),
    ("e3m2 mantissa width", "ldexp((double)(4 + f), e - 5)", "ldexp((double)(4 + f), e - 4)"),
    ("e3m2 subnormal scale", "ldexp((double)f, -4); /* f/4 * 2^-2 */", "ldexp((double)f, -3); /* f/4 * 2^-2 */"),
    ("fp6 bits straddling a byte dropped at shift 4", "if (shift > 2)", "if (shift > 4)"),
    ("fp6 elements a byte apart", "int64_t bit = 6 * idx;", "int64_t bit = 8 * idx;"),
    ("fp6 sign bit taken from the exponent", "int s = (c >> 5) & 1, e = (c >> 2) & 7", "int s = (c >> 4) & 1, e = (c >> 2) & 7"),
]

# Mistakes planted in the comparison (oracle/compare.py), caught by
# tests/test_compare.py: (description, text, replacement).
COMPARE_MUTANTS = [
    ("per-tensor scale applied twice on a block-scaled operand",
     "return float(np.abs(vals).max()) * per_tensor", "return float(np.abs(vals).max()) * per_tensor * per_tensor"),
    ("block scales not applied", "vals = vals.reshape(rows, w.k // 32, 32) * scales[:, :, None]",
     "vals = vals.reshape(rows, w.k // 32, 32) * 1.0"),
    ("per-tensor fp8 scale ignored",
     'per_tensor = (w.a_scale if which == "a" else w.b_scale) if fmt in ("e4m3", "e5m2") else 1.0',
     "per_tensor = 1.0"),
    ("M-major operand read as if K-major", "return vals[:rows, : w.k] if kmajor else vals[: w.k, :rows].T",
     "return vals[:rows, : w.k] if True else vals"),
    ("operand B's maximum taken from A", 'raw = w.a if which == "a" else w.b', "raw = w.a"),
    ("scale padding read as blocks", "[:rows, : w.k // 32]", "[:rows, : w.k // 32 + 1][:, 1:]"),
    ("gelu factor dropped", 'g = 1.13 if act == "gelu" else 1.0', "g = 1.0"),
    ("alpha dropped", "* k * abs(alpha) *", "* k *"),
    ("K dropped", "term = 2.0 ** -20 * k *", "term = 2.0 ** -20 *"),
    ("ulp one bit too fine", "(e - (p - 1))", "(e - p)"),
    ("subnormal spacing ignored", "e = np.maximum(np.where(a > 0, e, emin), emin)", "e = np.where(a > 0, e, emin)"),
]


def _run_mutant(case):
    desc, old, new = case
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not unique: {desc}"
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "oracle_mutant.c")
        lib = os.path.join(tmp, "liboracle_mutant.so")
        with open(src, "w") as f:
            f.write(text.replace(old, new))
        oracle.build(force=True, src=src, out=lib)
        env = dict(os.environ, THL_ORACLE_LIB_OVERRIDE=lib)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        return desc, r.returncode


def _run_compare_mutant(case):
    """Copy the oracle package, the generators and the comparison pins into a
    temporary tree, plant the mistake in its compare.py, and run the pins
    there (the built oracle library is reused)."""
    desc, old, new = case
    src = os.path.join(ROOT, "oracle", "compare.py")
    text = open(src).read()
    assert text.count(old) == 1, f"mutation anchor not unique: {desc}"
    with tempfile.TemporaryDirectory() as tmp:
        shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(tmp, "oracle"),
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
        shutil.copytree(os.path.join(ROOT, "workloads"), os.path.join(tmp, "workloads"),
                        ignore=shutil.ignore_patterns("__pycache__"))
        os.makedirs(os.path.join(tmp, "tests"))
        for name in ("conftest.py", "test_compare.py"):
            shutil.copy(os.path.join(ROOT, "tests", name), os.path.join(tmp, "tests", name))
        with open(os.path.join(tmp, "oracle", "compare.py"), "w") as f:
            f.write(text.replace(old, new))
        env = dict(os.environ, THL_ORACLE_LIB_OVERRIDE=oracle.build(force=False))
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(tmp, "tests", "test_compare.py")],
                           cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
        return desc, r.returncode


def test_unmutated_copies_pass_the_pins():
    # Control: the same machinery with the anchor replaced by itself must
    # pass, so that a mutant's failure means a pin caught it.
    assert _run_mutant(("control", MUTANTS[0][1], MUTANTS[0][1]))[1] == 0
    assert _run_compare_mutant(("control", COMPARE_MUTANTS[0][1], COMPARE_MUTANTS[0][1]))[1] == 0


def test_every_planted_mistake_fails_a_pin():
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_mutant, MUTANTS))
    survivors = [desc for desc, rc in results if rc == 0]
    assert not survivors, f"mutants that pass every pin: {survivors}"


def test_every_planted_comparison_mistake_fails_a_pin():
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_compare_mutant, COMPARE_MUTANTS))
    survivors = [desc for desc, rc in results if rc == 0]
    assert not survivors, f"mutants that pass every pin: {survivors}"
