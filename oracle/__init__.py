"""The CPU oracle for the fused-epilogue GEMM (ctypes binding of oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library never links or loads it, and the two share no code.

The oracle evaluates, element by element and in fp64 (int64 for int8),

    D(i,j) = act(alpha * s_a * s_b * sum_p a'(i,p) b'(p,j) + beta*C(i,j) + bias(i))

with a'(i,p) = A(i,p) * SFA(i, p // 32) for block-scaled operands.  The surface
and storage convention come from the "CUTLASS" knowledge-base page (opening
section and "Epilogues"); the block-scaled sum and the formats from
"Technical Documentation: NVIDIA/cutlass", section "Blackwell SM100 GEMMs"
("Block Scaled GEMMs" and the narrow-precision type tables).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Test hook: the pins' mutation test points this at a deliberately broken build.
_LIB_OVERRIDE = os.environ.get("THL_ORACLE_LIB_OVERRIDE")

TYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "i32": 4, "e4m3": 5, "e2m1": 6, "e8m0": 7, "e5m2": 9,
              "e2m3": 10, "e3m2": 11}
ACT_CODES = {"none": 0, "relu": 1, "gelu": 2}


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile liboracle.so with gcc -O2 -fopenmp (no fast-math)."""
    if _LIB_OVERRIDE and out == _LIB:
        return _LIB_OVERRIDE
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
             src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [
        ("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("a", ctypes.c_void_p), ("lda", ctypes.c_int64), ("op_a", ctypes.c_int32),
        ("type_a", ctypes.c_int32),
        ("b", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("op_b", ctypes.c_int32),
        ("type_b", ctypes.c_int32),
        ("c", ctypes.c_void_p), ("ldc", ctypes.c_int64), ("type_c", ctypes.c_int32),
        ("type_bias", ctypes.c_int32), ("bias", ctypes.c_void_p),
        ("alpha", ctypes.c_double), ("beta", ctypes.c_double),
        ("a_scale", ctypes.c_double), ("b_scale", ctypes.c_double),
        ("sfa", ctypes.c_void_p), ("ld_sfa", ctypes.c_int64),
        ("sfb", ctypes.c_void_p), ("ld_sfb", ctypes.c_int64),
        ("act", ctypes.c_int32), ("block", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        lib.oracle_gemm_elements.argtypes = [
            ctypes.POINTER(_Problem), ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_gemm_elements.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_mx_quantize.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_void_p]
        lib.oracle_mx_quantize.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(arr):
    if arr is None:
        return None
    assert isinstance(arr, np.ndarray) and arr.flags["C_CONTIGUOUS"], "host numpy buffers only"
    return arr.ctypes.data


def decode(type_name: str, raw: np.ndarray, count: int | None = None) -> np.ndarray:
    """Decode ``count`` stored elements of ``raw`` (its bytes) to exact float64."""
    raw = np.ascontiguousarray(raw)
    if count is None:
        if type_name == "e2m1":
            count = raw.nbytes * 2
        elif type_name in ("e2m3", "e3m2"):
            count = raw.nbytes * 8 // 6
        else:
            count = raw.size
    out = np.empty(count, dtype=np.float64)
    rc = _load().oracle_decode(TYPE_CODES[type_name], _ptr(raw), count, _ptr(out))
    if rc != 0:
        raise ValueError(type_name)
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def gemm_elements(prob: dict, rows, cols, nthreads: int = 0) -> np.ndarray:
    """Evaluate D at (rows[t], cols[t]).

    ``prob`` keys: m, n, k; a, lda, op_a ('N'|'T'), type_a; b, ldb, op_b, type_b;
    optional c, ldc, type_c, beta; bias, type_bias; alpha; a_scale, b_scale;
    sfa, ld_sfa, sfb, ld_sfb; act ('none'|'relu'|'gelu').  Buffers are host
    numpy arrays holding the stored bits (leading dimensions in elements).
    Returns float64 values, or int64 for int8 x int8.
    """
    lib = _load()
    keep = []

    def buf(name):
        arr = prob.get(name)
        if arr is None:
            return None
        arr = np.ascontiguousarray(arr)
        keep.append(arr)
        return _ptr(arr)

    p = _Problem()
    p.m, p.n, p.k = int(prob["m"]), int(prob["n"]), int(prob["k"])
    p.a, p.lda = buf("a"), int(prob["lda"])
    p.op_a, p.type_a = (1 if prob["op_a"] == "T" else 0), TYPE_CODES[prob["type_a"]]
    p.b, p.ldb = buf("b"), int(prob["ldb"])
    p.op_b, p.type_b = (1 if prob["op_b"] == "T" else 0), TYPE_CODES[prob["type_b"]]
    p.beta = float(prob.get("beta", 0.0))
    p.c = buf("c") if p.beta != 0.0 else None
    p.ldc = int(prob.get("ldc", max(1, p.m)))
    p.type_c = TYPE_CODES[prob.get("type_c", "f32")]
    p.bias = buf("bias")
    p.type_bias = TYPE_CODES[prob.get("type_bias", "f32")]
    p.alpha = float(prob.get("alpha", 1.0))
    p.a_scale = float(prob.get("a_scale", 1.0))
    p.b_scale = float(prob.get("b_scale", 1.0))
    p.sfa, p.ld_sfa = buf("sfa"), int(prob.get("ld_sfa", 0))
    p.sfb, p.ld_sfb = buf("sfb"), int(prob.get("ld_sfb", 0))
    p.act = ACT_CODES[prob.get("act", "none")]
    p.block = int(prob.get("block", 32))
    if p.beta != 0.0 and p.c is None:
        raise ValueError("beta != 0 needs C")

    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    assert rows.shape == cols.shape
    integer = prob["type_a"] == "i8" and prob["type_b"] == "i8"
    out = np.empty(rows.size, dtype=np.int64 if integer else np.float64)
    rc = lib.oracle_gemm_elements(
        ctypes.byref(p), rows.size, _ptr(rows), _ptr(cols),
        None if integer else _ptr(out), _ptr(out) if integer else None, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the request")
    return out


def gemm_full(prob: dict, nthreads: int = 0) -> np.ndarray:
    """Every element of D, as an (m, n) array indexed [i, j]."""
    m, n = int(prob["m"]), int(prob["n"])
    jj, ii = np.meshgrid(np.arange(n), np.arange(m))
    return gemm_elements(prob, ii.ravel(), jj.ravel(), nthreads).reshape(m, n)


def mx_quantize_block(values, fmt: str):
    """OCP MX quantization of one block (1 .. 32 values) to ``fmt`` ('e2m1',
    'e4m3' or 'e5m2'): returns (element codes as a uint8 array, E8M0 scale
    code)."""
    vals = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    codes = np.zeros(vals.size, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.uint8)
    rc = _load().oracle_mx_quantize(TYPE_CODES[fmt], _ptr(vals), vals.size, _ptr(codes), _ptr(scale))
    if rc != 0:
        raise ValueError("oracle rejected the block")
    return codes, int(scale[0])


def mx_quantize_columns(y, fmt: str, block: int = 32):
    """MX output of an (m, n) array of values: each column cut into blocks of
    ``block`` consecutive rows (the last possibly shorter), each block
    quantized by mx_quantize_block.  Returns (codes (m, n) uint8, scales
    (ceil(m/block), n) uint8)."""
    y = np.asarray(y, dtype=np.float64)
    m, n = y.shape
    nb = (m + block - 1) // block
    codes = np.zeros((m, n), dtype=np.uint8)
    scales = np.zeros((nb, n), dtype=np.uint8)
    for j in range(n):
        for b in range(nb):
            c, s = mx_quantize_block(y[b * block: (b + 1) * block, j], fmt)
            codes[b * block: b * block + c.size, j] = c
            scales[b, j] = s
    return codes, scales
