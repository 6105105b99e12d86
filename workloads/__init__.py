"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random numbers and encodes them into the stored bit
patterns of each operand format; it holds none of the GEMM's arithmetic.  Both
the GPU path (via ``bench.py`` and the tests) and the CPU oracle read the same
host buffers it returns.  Every tensor comes from its own numpy PCG64 stream
keyed by (seed, tensor id): A=1, B=2, C=3, bias=4, output sample=5.

Storage follows the BLAS column-major convention with op in {N, T}: a stored
r x c matrix with leading dimension ld occupies c rows of ld elements in
memory.  For A, op N stores op(A) (M x K) itself and op T stores its transpose;
likewise for B with op(B) (K x N).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

TENSOR_IDS = {"a": 1, "b": 2, "c": 3, "bias": 4, "sample": 5}

# Bytes per element of each stored format (fp4 packs two per byte).
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "i32": 4, "e4m3": 1, "e5m2": 1, "e2m1": 0.5, "e2m3": 0.75,
              "e3m2": 0.75}


def rng(seed: int, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), TENSOR_IDS[tensor]]))


# ----------------------------------------------------------------- encoders

def encode(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round float64 values to ``fmt`` (round-to-nearest-even) and return the
    stored bits: uint16 for f16/bf16, uint32 for f32, uint8 for e4m3/e5m2, int8 and
    int32 for the integer formats (values must already be integral)."""
    if fmt == "f32":
        return x.astype(np.float32).view(np.uint32)
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    if fmt == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    if fmt == "e4m3":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
        return t.view(torch.uint8).numpy()
    if fmt == "e5m2":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e5m2)
        return t.view(torch.uint8).numpy()
    if fmt == "i8":
        return x.astype(np.int8)
    if fmt == "i32":
        return x.astype(np.int32)
    raise ValueError(fmt)


# OCP E2M1 magnitudes by code 0..7, and the midpoints between neighbours.
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def encode_e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Round to the nearest E2M1 value, ties to the even code, saturating at
    +-6; returns one 4-bit code per element (uint8)."""
    a = np.abs(v)
    code = np.zeros(v.shape, dtype=np.uint8)
    for c, t in enumerate(_E2M1_MID):
        up = (a > t) | ((a == t) & (c % 2 == 1))  # a tie goes to the even code
        code += up.astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def mx_quantize(x: np.ndarray, block: int = 32):
    """OCP MX quantization of rows of ``x`` (shape R x K, K % block == 0):
    per block the shared exponent is floor(log2(amax)) - 2 (2 is E2M1's largest
    exponent), clamped to [-127, 127]; elements are x / 2^X rounded to E2M1.
    Returns (codes R x K uint8, scale codes R x K/block uint8)."""
    r, k = x.shape
    xb = x.reshape(r, k // block, block)
    amax = np.abs(xb).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2
    e = np.clip(e, -127, 127)
    e = np.where(amax > 0, e, -127)
    codes = encode_e2m1_codes(xb / np.ldexp(1.0, e.astype(np.int64))[:, :, None])
    return codes.reshape(r, k), (e + 127).astype(np.uint8)


# Largest exponent and largest finite magnitude of the OCP fp8 formats.
_FP8_EMAX = {"e4m3": (8, 448.0), "e5m2": (15, 57344.0)}


def mx_quantize_fp8(x: np.ndarray, fmt: str = "e4m3", block: int = 32):
    """OCP MX quantization of rows of ``x`` (R x K, K % block == 0) to an fp8
    format: per block the shared exponent is floor(log2(amax)) - emax (emax
    is the format's largest exponent: 8 for E4M3, 15 for E5M2), clamped to
    [-127, 127]; elements are x / 2^X rounded to the format (RNE; the block's
    largest lands below 2^(emax+1), so values past the largest finite
    magnitude are clamped to it first).  Returns (codes R x K uint8, scale
    codes R x K/block uint8)."""
    emax, top = _FP8_EMAX[fmt]
    r, k = x.shape
    xb = x.reshape(r, k // block, block)
    amax = np.abs(xb).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - emax
    e = np.clip(e, -127, 127)
    e = np.where(amax > 0, e, -127)
    y = np.clip(xb / np.ldexp(1.0, e.astype(np.int64))[:, :, None], -top, top)
    return encode(y.reshape(r, k), fmt), (e + 127).astype(np.uint8)


def mx_quantize_e4m3(x: np.ndarray, block: int = 32):
    """mx_quantize_fp8 with E4M3 elements."""
    return mx_quantize_fp8(x, "e4m3", block)


# OCP fp6 formats: (exponent bits, mantissa bits, largest exponent); bias
# 2^(e-1) - 1, every code finite.
_FP6 = {"e2m3": (2, 3, 2), "e3m2": (3, 2, 4)}


def _fp6_magnitudes(fmt: str) -> np.ndarray:
    """Magnitude of each non-negative fp6 code 0 .. 31, in code order."""
    e_bits, m_bits, _ = _FP6[fmt]
    bias = 2 ** (e_bits - 1) - 1
    out = []
    for c in range(32):
        e, f = c >> m_bits, c & ((1 << m_bits) - 1)
        frac = f / 2 ** m_bits
        out.append(frac * 2.0 ** (1 - bias) if e == 0 else (1 + frac) * 2.0 ** (e - bias))
    return np.array(out)


def encode_fp6_codes(v: np.ndarray, fmt: str) -> np.ndarray:
    """Round to the nearest value of an fp6 format (E2M3 or E3M2), ties to the
    even code, saturating at the largest magnitude; one 6-bit code per
    element (uint8, sign in bit 5)."""
    mags = _fp6_magnitudes(fmt)
    mid = (mags[1:] + mags[:-1]) / 2
    a = np.abs(v)
    idx = np.searchsorted(mid, a, side="left")
    at = np.minimum(idx, mid.size - 1)
    idx = idx + ((idx < mid.size) & (a == mid[at]) & (idx % 2 == 1))
    return (idx.astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 5)).astype(np.uint8)


def mx_quantize_fp6(x: np.ndarray, fmt: str, block: int = 32):
    """OCP MX quantization of rows of ``x`` (R x K, K % block == 0) to an fp6
    format: shared exponent floor(log2(amax)) - emax (2 for E2M3, 4 for E3M2),
    clamped to [-127, 127]; elements x / 2^X rounded to the format.  Returns
    (codes R x K uint8, scale codes R x K/block uint8)."""
    emax = _FP6[fmt][2]
    r, k = x.shape
    xb = x.reshape(r, k // block, block)
    amax = np.abs(xb).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - emax
    e = np.clip(e, -127, 127)
    e = np.where(amax > 0, e, -127)
    codes = encode_fp6_codes(xb / np.ldexp(1.0, e.astype(np.int64))[:, :, None], fmt)
    return codes.reshape(r, k), (e + 127).astype(np.uint8)


# ----------------------------------------------------------------- storage

def store_colmajor(s: np.ndarray, ld: int) -> np.ndarray:
    """Column-major storage of the r x c matrix ``s`` with leading dimension
    ld: a (c, ld) array whose row j holds column j; padding is zero."""
    r, c = s.shape
    assert ld >= max(1, r)
    mem = np.zeros((c, ld), dtype=s.dtype)
    mem[:, :r] = s.T
    return mem


def pack_e2m1(mem_codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along the contiguous dimension, the even element in
    the low nibble."""
    assert mem_codes.shape[-1] % 2 == 0
    return (mem_codes[..., 0::2] | (mem_codes[..., 1::2] << 4)).astype(np.uint8)


def pack_fp6(mem_codes: np.ndarray) -> np.ndarray:
    """Four 6-bit codes in three bytes along the contiguous dimension: element
    t in bits 6t .. 6t+5 of the little-endian bit stream."""
    n = mem_codes.shape[-1]
    assert n % 4 == 0
    c = mem_codes.astype(np.uint32).reshape(*mem_codes.shape[:-1], n // 4, 4)
    w = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)
    out = np.stack([w & 255, (w >> 8) & 255, (w >> 16) & 255], axis=-1)
    return out.reshape(*mem_codes.shape[:-1], n // 4 * 3).astype(np.uint8)


def stored_shape(rows: int, cols: int, op: str, which: str):
    """(r, c) of the stored matrix for logical op(X) of shape rows x cols."""
    return (rows, cols) if op == "N" else (cols, rows)


# ----------------------------------------------------------------- workloads

@dataclass
class Workload:
    """Host buffers (stored bits) and the scalar parameters of one GEMM."""
    name: str
    m: int
    n: int
    k: int
    type_a: str
    type_b: str
    type_d: str
    op_a: str
    op_b: str
    lda: int
    ldb: int
    ldd: int
    a: np.ndarray
    b: np.ndarray
    alpha: float = 1.0
    beta: float = 0.0
    c: np.ndarray | None = None
    ldc: int = 0
    type_c: str = "f32"
    bias: np.ndarray | None = None
    type_bias: str = "f32"
    act: str = "none"
    a_scale: float = 1.0
    b_scale: float = 1.0
    sfa: np.ndarray | None = None
    ld_sfa: int = 0
    sfb: np.ndarray | None = None
    ld_sfb: int = 0
    seed: int = 0
    extra: dict = field(default_factory=dict)

    def oracle_problem(self) -> dict:
        return dict(m=self.m, n=self.n, k=self.k, a=self.a, lda=self.lda, op_a=self.op_a,
                    type_a=self.type_a, b=self.b, ldb=self.ldb, op_b=self.op_b,
                    type_b=self.type_b, c=self.c, ldc=self.ldc or max(1, self.m),
                    type_c=self.type_c, beta=self.beta, bias=self.bias,
                    type_bias=self.type_bias, alpha=self.alpha, a_scale=self.a_scale,
                    b_scale=self.b_scale, sfa=self.sfa, ld_sfa=self.ld_sfa, sfb=self.sfb,
                    ld_sfb=self.ld_sfb, act=self.act)

    def flops(self) -> int:
        return 2 * self.m * self.n * self.k

    def sample(self, count: int = 4096):
        """`count` distinct output positions, uniform without replacement."""
        total = self.m * self.n
        g = rng(self.seed, "sample")
        if total <= count:
            idx = np.arange(total, dtype=np.int64)
        else:
            idx = g.choice(total, size=count, replace=False).astype(np.int64)
        return idx % self.m, idx // self.m


def _uniform(g, shape):
    return g.uniform(-1.0, 1.0, size=shape)


def _operand(x_logical: np.ndarray, fmt: str, op: str, ld: int):
    return store_colmajor(encode(x_logical if op == "N" else x_logical.T, fmt), ld)


def make(kind: str, m: int, n: int, k: int, seed: int | None = None, *, op_a=None, op_b=None,
         lda=None, ldb=None, ldd=None, ldc=None, act=None, bias=None, beta=None,
         type_d=None, type_c=None, type_bias=None, alpha=1.0) -> Workload:
    """Build one of the five workload kinds at shape m x n x k.

    kinds: 'fp16'  fp16 T/N, U[-1,1], fp32 out, D = A.B
           'bf16'  bf16 N/N, U[-1,1] A, B, C, bias, bf16 out, D = relu(A.B + C + bias[m])
           'int8'  int8 T/N, uniform integers in [-128,127], int32 out, D = A.B
           'fp8'   e4m3 T/N, N(0,1) scaled per tensor to +-448, bf16 out, D = s_a s_b A.B
           'fp8e5m2' e5m2 T/N, N(0,1) scaled per tensor to +-57344, otherwise as 'fp8'
           'fp8e4e5', 'fp8e5e4'  e4m3 A with e5m2 B, and the other way round
           'mxfp4' e2m1 T/N, N(0,1) MX-quantized per 32 K-elements, C bf16 N(0,1),
                   bf16 out, D = A.B + C
           'mxfp8' e4m3 T/N, N(0,1) MX-quantized per 32 K-elements, bf16 out, D = A.B
           'mxfp8e5m2' the same with e5m2 elements; 'mxfp8e4e5', 'mxfp8e5e4' e4m3 A with
                   e5m2 B, and the other way round
    Keyword overrides change ops, leading dimensions, the epilogue and the
    float C, D and bias types for the edge-case sweeps."""
    defaults = {
        "fp16": dict(seed=1001, op_a="T", op_b="N", type_ab="f16", type_d="f32"),
        "bf16": dict(seed=1002, op_a="N", op_b="N", type_ab="bf16", type_d="bf16"),
        "int8": dict(seed=1003, op_a="T", op_b="N", type_ab="i8", type_d="i32"),
        "fp8": dict(seed=1004, op_a="T", op_b="N", type_ab="e4m3", type_d="bf16"),
        "fp8e5m2": dict(seed=1006, op_a="T", op_b="N", type_ab="e5m2", type_d="bf16"),
        "fp8e4e5": dict(seed=1008, op_a="T", op_b="N", type_ab="e4m3", type_b="e5m2", type_d="bf16"),
        "fp8e5e4": dict(seed=1009, op_a="T", op_b="N", type_ab="e5m2", type_b="e4m3", type_d="bf16"),
        "mxfp4": dict(seed=1005, op_a="T", op_b="N", type_ab="e2m1", type_d="bf16"),
        "mxfp8": dict(seed=1007, op_a="T", op_b="N", type_ab="e4m3", type_d="bf16"),
        "mxfp8e5m2": dict(seed=1010, op_a="T", op_b="N", type_ab="e5m2", type_d="bf16"),
        "mxfp8e4e5": dict(seed=1011, op_a="T", op_b="N", type_ab="e4m3", type_b="e5m2", type_d="bf16"),
        "mxfp8e5e4": dict(seed=1012, op_a="T", op_b="N", type_ab="e5m2", type_b="e4m3", type_d="bf16"),
    }[kind]
    seed = defaults["seed"] if seed is None else seed
    op_a = op_a or defaults["op_a"]
    op_b = op_b or defaults["op_b"]
    fmt = defaults["type_ab"]
    fmt_b = defaults.get("type_b", fmt)
    type_d = type_d or defaults["type_d"]
    ra, ca = stored_shape(m, k, op_a, "a")
    rb, cb = stored_shape(k, n, op_b, "b")
    lda = lda or max(1, ra)
    ldb = ldb or max(1, rb)
    ldd = ldd or max(1, m)
    ga, gb, gc, gbias = rng(seed, "a"), rng(seed, "b"), rng(seed, "c"), rng(seed, "bias")
    w = dict(name=kind, m=m, n=n, k=k, type_a=fmt, type_b=fmt_b, type_d=type_d, op_a=op_a,
             op_b=op_b, lda=lda, ldb=ldb, ldd=ldd, seed=seed, alpha=alpha)

    if kind in ("fp16", "bf16"):
        xa, xb = _uniform(ga, (m, k)), _uniform(gb, (k, n))
        w["a"], w["b"] = _operand(xa, fmt, op_a, lda), _operand(xb, fmt, op_b, ldb)
        if kind == "bf16":
            use_c = True if beta is None else beta != 0.0
            w["beta"] = 1.0 if beta is None else beta
            if use_c:
                ldc = ldc or max(1, m)
                tc = type_c or "bf16"
                w["c"], w["ldc"], w["type_c"] = store_colmajor(encode(_uniform(gc, (m, n)), tc), ldc), ldc, tc
            w["act"] = "relu" if act is None else act
            if bias is None or bias:
                tb = type_bias or "bf16"
                w["bias"], w["type_bias"] = encode(_uniform(gbias, (m,)), tb), tb
        else:
            w["beta"] = 0.0 if beta is None else beta
            if w["beta"] != 0.0:
                ldc = ldc or max(1, m)
                tc = type_c or "f32"
                w["c"], w["ldc"], w["type_c"] = store_colmajor(encode(_uniform(gc, (m, n)), tc), ldc), ldc, tc
            w["act"] = act or "none"
            if bias:
                tb = type_bias or "f32"
                w["bias"], w["type_bias"] = encode(_uniform(gbias, (m,)), tb), tb
    elif kind == "int8":
        xa = ga.integers(-128, 128, size=(m, k)).astype(np.float64)
        xb = gb.integers(-128, 128, size=(k, n)).astype(np.float64)
        w["a"], w["b"] = _operand(xa, "i8", op_a, lda), _operand(xb, "i8", op_b, ldb)
        w["beta"] = 0.0 if beta is None else beta
        if w["beta"] != 0.0:
            ldc = ldc or max(1, m)
            w["c"], w["ldc"], w["type_c"] = store_colmajor(
                gc.integers(-1000, 1000, size=(m, n)).astype(np.int32), ldc), ldc, "i32"
        w["act"] = act or "none"
        if bias:
            w["bias"], w["type_bias"] = gbias.integers(-1000, 1000, size=(m,)).astype(np.int32), "i32"
    elif kind in ("fp8", "fp8e5m2", "fp8e4e5", "fp8e5e4"):
        top = {"e4m3": 448.0, "e5m2": 57344.0}  # each format's largest finite magnitude
        xa, xb = ga.standard_normal((m, k)), gb.standard_normal((k, n))
        sa = float(np.abs(xa).max()) / top[fmt] if xa.size else 1.0
        sb = float(np.abs(xb).max()) / top[fmt_b] if xb.size else 1.0
        sa, sb = float(np.float32(sa or 1.0)), float(np.float32(sb or 1.0))
        w["a"], w["b"] = _operand(xa / sa, fmt, op_a, lda), _operand(xb / sb, fmt_b, op_b, ldb)
        w["a_scale"], w["b_scale"] = sa, sb
        w["beta"] = 0.0 if beta is None else beta
        if w["beta"] != 0.0:
            ldc = ldc or max(1, m)
            tc = type_c or "bf16"
            w["c"], w["ldc"], w["type_c"] = store_colmajor(encode(gc.standard_normal((m, n)), tc), ldc), ldc, tc
        w["act"] = act or "none"
        if bias:
            tb = type_bias or "bf16"
            w["bias"], w["type_bias"] = encode(gbias.standard_normal(m), tb), tb
    elif kind == "mxfp4":
        assert op_a == "T" and op_b == "N", "MX blocks run along the contiguous K"
        assert k % 32 == 0
        xa, xb = ga.standard_normal((m, k)), gb.standard_normal((n, k))  # B drawn as its stored N x K
        ca_codes, w["sfa"] = mx_quantize(xa) if k else (np.zeros((m, 0), np.uint8), np.zeros((m, 0), np.uint8))
        cb_codes, w["sfb"] = mx_quantize(xb) if k else (np.zeros((n, 0), np.uint8), np.zeros((n, 0), np.uint8))
        # scale rows padded to a multiple of 16 bytes (the kernels copy 16-byte groups)
        ld_sf = max(16, (k // 32 + 15) // 16 * 16)
        w["ld_sfa"] = w["ld_sfb"] = ld_sf
        pad_a = np.full((m, ld_sf), 127, np.uint8)
        pad_a[:, : k // 32] = w["sfa"]
        pad_b = np.full((n, ld_sf), 127, np.uint8)
        pad_b[:, : k // 32] = w["sfb"]
        w["sfa"], w["sfb"] = pad_a, pad_b
        mem_a = np.zeros((m, lda), np.uint8)
        mem_a[:, :k] = ca_codes
        mem_b = np.zeros((n, ldb), np.uint8)
        mem_b[:, :k] = cb_codes
        w["a"], w["b"] = pack_e2m1(mem_a), pack_e2m1(mem_b)
        w["beta"] = 1.0 if beta is None else beta
        if w["beta"] != 0.0:
            ldc = ldc or max(1, m)
            tc = type_c or "bf16"
            w["c"], w["ldc"], w["type_c"] = store_colmajor(encode(gc.standard_normal((m, n)), tc), ldc), ldc, tc
        w["act"] = act or "none"
        if bias:
            tb = type_bias or "bf16"
            w["bias"], w["type_bias"] = encode(gbias.standard_normal(m), tb), tb
    elif kind in ("mxfp8", "mxfp8e5m2", "mxfp8e4e5", "mxfp8e5e4"):
        assert op_a == "T" and op_b == "N", "MX blocks run along the contiguous K"
        assert k % 32 == 0
        xa, xb = ga.standard_normal((m, k)), gb.standard_normal((n, k))  # B drawn as its stored N x K
        ca, w["sfa"] = mx_quantize_fp8(xa, fmt) if k else (np.zeros((m, 0), np.uint8), np.zeros((m, 0), np.uint8))
        cb, w["sfb"] = mx_quantize_fp8(xb, fmt_b) if k else (np.zeros((n, 0), np.uint8), np.zeros((n, 0), np.uint8))
        ld_sf = max(16, (k // 32 + 15) // 16 * 16)
        w["ld_sfa"] = w["ld_sfb"] = ld_sf
        pad_a = np.full((m, ld_sf), 127, np.uint8)
        pad_a[:, : k // 32] = w["sfa"]
        pad_b = np.full((n, ld_sf), 127, np.uint8)
        pad_b[:, : k // 32] = w["sfb"]
        w["sfa"], w["sfb"] = pad_a, pad_b
        mem_a = np.zeros((m, lda), np.uint8)
        mem_a[:, :k] = ca
        mem_b = np.zeros((n, ldb), np.uint8)
        mem_b[:, :k] = cb
        w["a"], w["b"] = mem_a, mem_b
        w["beta"] = 0.0 if beta is None else beta
        if w["beta"] != 0.0:
            ldc = ldc or max(1, m)
            tc = type_c or "bf16"
            w["c"], w["ldc"], w["type_c"] = store_colmajor(encode(gc.standard_normal((m, n)), tc), ldc), ldc, tc
        w["act"] = act or "none"
        if bias:
            tb = type_bias or "bf16"
            w["bias"], w["type_bias"] = encode(gbias.standard_normal(m), tb), tb
    else:
        raise ValueError(kind)
    return Workload(**w)


# ------------------------------------------------------ narrow-format pairs

_LD_QUANTUM = {"e2m1": 2, "e2m3": 4, "e3m2": 4}  # elements a stored line is padded to (whole bytes)
_TOP = {"e4m3": 448.0, "e5m2": 57344.0}


def _narrow_codes(g, rows: int, k: int, fmt: str, mx: bool):
    """Codes (rows x k, uint8) of N(0,1) draws in ``fmt``: MX-quantized per 32
    K-elements (returns the scale codes too), or, without block scales, fp8
    scaled per tensor to its largest magnitude and fp4 / fp6 drawn in range."""
    x = g.standard_normal((rows, k))
    if mx:
        if fmt == "e2m1":
            return mx_quantize(x) + (1.0,)
        if fmt in _FP6:
            return mx_quantize_fp6(x, fmt) + (1.0,)
        return mx_quantize_fp8(x, fmt) + (1.0,)
    if fmt == "e2m1":
        return encode_e2m1_codes(2.0 * x), None, 1.0
    if fmt in _FP6:
        return encode_fp6_codes(2.0 * x if fmt == "e2m3" else 6.0 * x, fmt), None, 1.0
    s = float(np.float32((float(np.abs(x).max()) / _TOP[fmt]) or 1.0)) if x.size else 1.0
    return encode(x / s, fmt), None, s


def _store_lines(codes_rows: np.ndarray, kmajor: bool, ld: int, fmt: str) -> np.ndarray:
    """Stored bytes of an operand given as logical rows x K codes: K-major
    lines are the rows, otherwise the K-indices; packed for fp4 / fp6."""
    lines = codes_rows if kmajor else codes_rows.T
    mem = np.zeros((lines.shape[0], ld), np.uint8)
    mem[:, : lines.shape[1]] = lines
    if fmt == "e2m1":
        return pack_e2m1(mem)
    if fmt in _FP6:
        return pack_fp6(mem)
    return mem


def make_narrow(type_a: str, type_b: str, m: int, n: int, k: int, *, mx: bool, op_a: str = "T", op_b: str = "N",
                lda=None, ldb=None, seed: int = 1020, type_d: str = "bf16", beta: float = 0.0, act: str = "none",
                bias: bool = False, alpha: float = 1.0, ldd=None) -> Workload:
    """A GEMM over any pair of the 8-, 6- and 4-bit float formats (e4m3, e5m2,
    e2m3, e3m2, e2m1) in any layout: N(0,1) operands, MX-quantized per 32
    K-elements when ``mx`` (scale rows padded to 16 bytes with 127), else fp8
    per-tensor scaled and fp4 / fp6 in range; C (when beta != 0) and bias
    bf16 N(0,1)."""
    ga, gb, gc, gbias = rng(seed, "a"), rng(seed, "b"), rng(seed, "c"), rng(seed, "bias")
    ca, sfa, sa = _narrow_codes(ga, m, k, type_a, mx)
    cb, sfb, sb = _narrow_codes(gb, n, k, type_b, mx)
    a_km, b_km = op_a == "T", op_b == "N"
    qa, qb = _LD_QUANTUM.get(type_a, 1), _LD_QUANTUM.get(type_b, 1)
    lda = lda or max(qa, -(-(k if a_km else m) // qa) * qa)
    ldb = ldb or max(qb, -(-(k if b_km else n) // qb) * qb)
    w = dict(name=f"{'mx' if mx else ''}{type_a}x{type_b}", m=m, n=n, k=k, type_a=type_a, type_b=type_b,
             type_d=type_d, op_a=op_a, op_b=op_b, lda=lda, ldb=ldb, ldd=ldd or max(1, m), seed=seed, alpha=alpha,
             a=_store_lines(ca, a_km, lda, type_a), b=_store_lines(cb, b_km, ldb, type_b), a_scale=sa, b_scale=sb,
             beta=beta, act=act)
    if mx:
        ld_sf = max(16, (k // 32 + 15) // 16 * 16)
        pa = np.full((m, ld_sf), 127, np.uint8)
        pa[:, : k // 32] = sfa
        pb = np.full((n, ld_sf), 127, np.uint8)
        pb[:, : k // 32] = sfb
        w.update(sfa=pa, sfb=pb, ld_sfa=ld_sf, ld_sfb=ld_sf)
    if beta != 0.0:
        w.update(c=store_colmajor(encode(gc.standard_normal((m, n)), "bf16"), max(1, m)), ldc=max(1, m),
                 type_c="bf16")
    if bias:
        w.update(bias=encode(gbias.standard_normal(m), "bf16"), type_bias="bf16")
    return Workload(**w)
