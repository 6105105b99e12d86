"""Parity comparison between a GPU result and the oracle.

TEST INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the
benchmark's parity report).

The float bar: |D - y| <= 2^-20 * K * |alpha| * max|a'| * max|b'| * g + ulp_out(y)
where a', b' are the dequantized operands, g = 1.13 for GELU (a bound on
|gelu'|) and 1 otherwise, and ulp_out(y) is the spacing of the output format at
|y| (subnormal spacing below the smallest normal).  Integer outputs must match
exactly.  The operand-error term is the accumulation bound of the requested
fp32 accumulate; the ulp term covers the single round-to-nearest-even of the
stored result.
"""
from __future__ import annotations

import numpy as np

# (significand bits including the hidden one, minimum normal exponent)
_FORMATS = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}


def ulp_out(fmt: str, y) -> np.ndarray:
    """Spacing of format ``fmt`` at |y| (elementwise, float64)."""
    p, emin = _FORMATS[fmt]
    a = np.abs(np.asarray(y, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, emin), emin)
    # Guard against log2 landing one below an exact power of two.
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= a, e + 1, e)
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int64))


def float_tolerance(k: int, alpha: float, max_a: float, max_b: float, out_fmt: str, y,
                    act: str = "none") -> np.ndarray:
    g = 1.13 if act == "gelu" else 1.0
    term = 2.0 ** -20 * k * abs(alpha) * max_a * max_b * g
    return term + ulp_out(out_fmt, y)


def check_float(got, want, tol) -> dict:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bad = ~(err <= tol)  # NaN counts as bad
    worst = int(np.argmax(np.where(np.isfinite(err), err - tol, np.inf))) if err.size else 0
    return {"ok": not bool(bad.any()), "n_bad": int(bad.sum()), "n": int(err.size),
            "max_err": float(err[np.isfinite(err)].max()) if np.isfinite(err).any() else
            (float("nan") if err.size else 0.0),
            "worst_index": worst}


def check_exact(got, want) -> dict:
    got = np.asarray(got, dtype=np.int64)
    want = np.asarray(want, dtype=np.int64)
    bad = got != want
    return {"ok": not bool(bad.any()), "n_bad": int(bad.sum()), "n": int(got.size)}


def logical_operand(w, which: str) -> np.ndarray:
    """The operand as its logical rows x K matrix (A: m x k; B: n x k, one
    row per column of op(B)) of decoded element values, read from its storage
    (lines of ld elements along K, or along the rows, by op), before any
    scale."""
    from . import decode

    raw = w.a if which == "a" else w.b
    fmt = w.type_a if which == "a" else w.type_b
    ld = w.lda if which == "a" else w.ldb
    rows = w.m if which == "a" else w.n
    kmajor = (w.op_a == "T") if which == "a" else (w.op_b == "N")
    if raw.size == 0 or rows == 0 or w.k == 0:
        return np.zeros((rows, w.k))
    vals = decode(fmt, raw).reshape(-1, ld)
    return vals[:rows, : w.k] if kmajor else vals[: w.k, :rows].T


def operand_max_abs(w, which: str) -> float:
    """max |a'| (or |b'|) over the dequantized operand of a workload, decoded
    by the oracle's own decoders: per-tensor scale for fp8, per-32-block E8M0
    scale along K for the block-scaled formats, whatever the storage."""
    from . import decode

    fmt = w.type_a if which == "a" else w.type_b
    vals = logical_operand(w, which)
    if vals.size == 0:
        return 0.0
    per_tensor = (w.a_scale if which == "a" else w.b_scale) if fmt in ("e4m3", "e5m2") else 1.0
    if w.sfa is not None:  # block-scaled
        sf = w.sfa if which == "a" else w.sfb
        ld_sf = w.ld_sfa if which == "a" else w.ld_sfb
        rows = vals.shape[0]
        scales = decode("e8m0", np.ascontiguousarray(sf)).reshape(-1, ld_sf)[:rows, : w.k // 32]
        vals = vals.reshape(rows, w.k // 32, 32) * scales[:, :, None]
    return float(np.abs(vals).max()) * per_tensor


def parity_check(w, d_values, rows, cols, ref=None) -> dict:
    """Compare GPU outputs at (rows, cols) (already decoded to float64, or
    int64 for the integer path) against the oracle."""
    from . import gemm_elements

    if ref is None:
        ref = gemm_elements(w.oracle_problem(), rows, cols)
    if w.type_a == "i8":
        return check_exact(d_values, ref)
    tol = float_tolerance(w.k, w.alpha,
                          operand_max_abs(w, "a"), operand_max_abs(w, "b"), w.type_d, ref,
                          w.act)
    return check_float(d_values, ref, tol)
