"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (on the CPU, in a temporary
directory), builds it, and runs the pin suite against it; the suite must fail.
"""
import os
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


def test_every_planted_mistake_fails_a_pin():
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_mutant, MUTANTS))
    survivors = [desc for desc, rc in results if rc == 0]
    assert not survivors, f"mutants that pass every pin: {survivors}"
