"""Python binding of libthl.so: the MI355X tiled GEMM with a fused epilogue
and the Shape:Stride layout module.

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels, and the layout algebra in its C++.  The names match the C entry
points of ``include/thl.h``.  Importing this module fails loudly when the
built library is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libthl.so")

THL_OK, THL_ERR_INVALID, THL_ERR_UNSUPPORTED, THL_ERR_MISALIGNED, THL_ERR_HIP, THL_ERR_UNDEFINED = (
    0, -1, -2, -3, -4, -5)
THL_ERR_SCRATCH = -6
THL_OP_N, THL_OP_T = 0, 1
DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "i32": 4, "e4m3": 5, "e2m1": 6, "e8m0": 7, "none": 8, "e5m2": 9,
          "e2m3": 10, "e3m2": 11}
THL_EPI_NONE, THL_EPI_BIAS, THL_EPI_RELU, THL_EPI_GELU = 0, 1, 2, 4


class ThlError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {thl_status_string(status)} ({status})" if what else thl_status_string(status))


class thl_dtypes(ctypes.Structure):
    _fields_ = [("a", ctypes.c_int), ("b", ctypes.c_int), ("c", ctypes.c_int), ("d", ctypes.c_int),
                ("bias", ctypes.c_int), ("acc", ctypes.c_int)]


class thl_epilogue(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint), ("bias", ctypes.c_void_p), ("sfd", ctypes.c_void_p),
                ("ld_sfd", ctypes.c_int64)]


class thl_scales(ctypes.Structure):
    _fields_ = [("a_scale", ctypes.c_float), ("b_scale", ctypes.c_float), ("sfa", ctypes.c_void_p),
                ("ld_sfa", ctypes.c_int64), ("sfb", ctypes.c_void_p), ("ld_sfb", ctypes.c_int64)]


class thl_group_problem(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64),
                ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64), ("D", ctypes.c_void_p), ("ldd", ctypes.c_int64),
                ("bias", ctypes.c_void_p), ("sfa", ctypes.c_void_p), ("ld_sfa", ctypes.c_int64),
                ("sfb", ctypes.c_void_p), ("ld_sfb", ctypes.c_int64)]


def _load():
    # One HIP runtime per process.  torch ships its own libamdhip64 and asks
    # for it by its unversioned name, so loading libthl first (which pulls in
    # the system libamdhip64.so.7) would leave two runtimes in the process and
    # device pointers from one invalid in the other.  Importing torch first
    # makes libthl bind to torch's runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python tile_hierarchy_linear_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, cp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_char_p, ctypes.c_size_t
    p64 = ctypes.POINTER(ctypes.c_int64)
    lib.thl_gemm.argtypes = [i64, i64, i64, vp, i64, ctypes.c_int, vp, i64, ctypes.c_int, vp, i64, vp, i64,
                             ctypes.c_float, ctypes.c_float, ctypes.POINTER(thl_dtypes),
                             ctypes.POINTER(thl_epilogue), ctypes.POINTER(thl_scales), vp]
    lib.thl_gemm.restype = ctypes.c_int
    lib.thl_gemm_noalloc.argtypes = lib.thl_gemm.argtypes
    lib.thl_gemm_noalloc.restype = ctypes.c_int
    lib.thl_gemm_batched.argtypes = [i64, i64, i64, i64, vp, i64, i64, ctypes.c_int, vp, i64, i64, ctypes.c_int,
                                     vp, i64, i64, vp, i64, i64, ctypes.c_float, ctypes.c_float,
                                     ctypes.POINTER(thl_dtypes), ctypes.POINTER(thl_epilogue), i64,
                                     ctypes.POINTER(thl_scales), i64, i64, vp]
    lib.thl_gemm_batched.restype = ctypes.c_int
    lib.thl_gemm_grouped.argtypes = [i64, ctypes.POINTER(thl_group_problem), vp, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_float, ctypes.c_float, ctypes.POINTER(thl_dtypes),
                                     ctypes.POINTER(thl_epilogue), ctypes.POINTER(thl_scales), vp]
    lib.thl_gemm_grouped.restype = ctypes.c_int
    lib.thl_status_string.argtypes = [ctypes.c_int]
    lib.thl_status_string.restype = cp
    lib.thl_last_variant.restype = cp
    lib.thl_last_splits.restype = ctypes.c_int
    lib.thl_variant_count.restype = ctypes.c_int
    lib.thl_variant_name.argtypes = [ctypes.c_int]
    lib.thl_variant_name.restype = cp
    lib.thl_kernel_index_map.argtypes = [cp, p64, i64, p64, p64]
    lib.thl_kernel_index_map.restype = ctypes.c_int
    lib.thl_kernel_index_map_names.restype = cp
    for name in ("coalesce",):
        getattr(lib, "thl_layout_" + name).argtypes = [cp, ctypes.c_char_p, sz]
    for name in ("composition", "logical_divide", "zipped_divide", "tiled_divide", "flat_divide"):
        getattr(lib, "thl_layout_" + name).argtypes = [cp, cp, ctypes.c_char_p, sz]
    lib.thl_layout_complement.argtypes = [cp, i64, ctypes.c_char_p, sz]
    lib.thl_layout_local_tile.argtypes = [cp, cp, i64, p64, ctypes.c_char_p, sz]
    lib.thl_layout_local_partition.argtypes = [cp, cp, i64, p64, ctypes.c_char_p, sz]
    lib.thl_layout_eval.argtypes = [cp, p64, i64, p64]
    lib.thl_layout_eval_coord.argtypes = [cp, cp, p64]
    lib.thl_layout_info.argtypes = [cp, p64, p64, p64]
    lib.thl_layout_mode.argtypes = [cp, i64, ctypes.c_char_p, sz]
    lib.thl_swizzle_eval.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, cp, p64, i64, p64]
    return lib


_lib = _load()


def library():
    """The loaded ctypes library (for symbol checks)."""
    return _lib


# ------------------------------------------------------------------ status

def thl_status_string(status: int) -> str:
    return _lib.thl_status_string(int(status)).decode()


def thl_last_variant() -> str:
    return _lib.thl_last_variant().decode()


def thl_last_splits() -> int:
    return int(_lib.thl_last_splits())


def thl_variant_count() -> int:
    return int(_lib.thl_variant_count())


def thl_variant_name(i: int) -> str | None:
    r = _lib.thl_variant_name(int(i))
    return r.decode() if r else None


def variants() -> list[str]:
    return [thl_variant_name(i) for i in range(thl_variant_count())]


# ------------------------------------------------------------------ GEMM

def _dt(x) -> int:
    return DTYPES[x] if isinstance(x, str) else int(x)


def make_dtypes(a, b=None, c="f32", d="f32", bias="none", acc=None) -> thl_dtypes:
    b = a if b is None else b
    if acc is None:
        acc = "i32" if _dt(a) == DTYPES["i8"] else "f32"
    return thl_dtypes(_dt(a), _dt(b), _dt(c), _dt(d), _dt(bias), _dt(acc))


def thl_gemm(m, n, k, A, lda, opA, B, ldb, opB, C, ldc, D, ldd, alpha, beta, dtypes, epilogue=None,
             scales=None, stream=None) -> int:
    """Direct call of the C entry point.  Pointers are integers (device
    addresses) or None; opA/opB are THL_OP_N/THL_OP_T or 'N'/'T'; `stream` is
    a hipStream_t as an integer (torch: ``torch.cuda.current_stream().cuda_stream``).
    Returns the thl_status code."""
    opa = THL_OP_T if opA in ("T", THL_OP_T) else (THL_OP_N if opA in ("N", THL_OP_N) else int(opA))
    opb = THL_OP_T if opB in ("T", THL_OP_T) else (THL_OP_N if opB in ("N", THL_OP_N) else int(opB))
    return int(_lib.thl_gemm(int(m), int(n), int(k), A, int(lda), opa, B, int(ldb), opb, C, int(ldc), D,
                             int(ldd), float(alpha), float(beta), ctypes.byref(dtypes),
                             ctypes.byref(epilogue) if epilogue is not None else None,
                             ctypes.byref(scales) if scales is not None else None, stream))


def bind_thl_gemm(m, n, k, A, lda, opA, B, ldb, opB, C, ldc, D, ldd, alpha, beta, dtypes, epilogue=None,
                  scales=None, stream=None, entry="thl_gemm"):
    """The arguments of one thl_gemm (or thl_gemm_noalloc) call, marshalled
    once: returns a callable that issues exactly that call and returns its
    status.  For loops that repeat one call (timing), where rebuilding the
    ctypes arguments each time would cost more host time than a small
    kernel runs."""
    opa = THL_OP_T if opA in ("T", THL_OP_T) else (THL_OP_N if opA in ("N", THL_OP_N) else int(opA))
    opb = THL_OP_T if opB in ("T", THL_OP_T) else (THL_OP_N if opB in ("N", THL_OP_N) else int(opB))
    fn = getattr(_lib, entry)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    args = (i64(m), i64(n), i64(k), vp(A), i64(lda), ctypes.c_int(opa), vp(B), i64(ldb), ctypes.c_int(opb), vp(C),
            i64(ldc), vp(D), i64(ldd), ctypes.c_float(alpha), ctypes.c_float(beta), ctypes.byref(dtypes),
            ctypes.byref(epilogue) if epilogue is not None else None,
            ctypes.byref(scales) if scales is not None else None, vp(stream))
    keep = (dtypes, epilogue, scales)

    def call() -> int:
        return fn(*args)

    call.keep = keep  # the structures the byref arguments point into
    return call


def thl_gemm_noalloc(m, n, k, A, lda, opA, B, ldb, opB, C, ldc, D, ldd, alpha, beta, dtypes, epilogue=None,
                     scales=None, stream=None) -> int:
    """Direct call of the no-allocation C entry point (arguments as for thl_gemm)."""
    opa = THL_OP_T if opA in ("T", THL_OP_T) else (THL_OP_N if opA in ("N", THL_OP_N) else int(opA))
    opb = THL_OP_T if opB in ("T", THL_OP_T) else (THL_OP_N if opB in ("N", THL_OP_N) else int(opB))
    return int(_lib.thl_gemm_noalloc(int(m), int(n), int(k), A, int(lda), opa, B, int(ldb), opb, C, int(ldc), D,
                                     int(ldd), float(alpha), float(beta), ctypes.byref(dtypes),
                                     ctypes.byref(epilogue) if epilogue is not None else None,
                                     ctypes.byref(scales) if scales is not None else None, stream))


def thl_gemm_batched(batch, m, n, k, A, lda, stride_a, opA, B, ldb, stride_b, opB, C, ldc, stride_c, D, ldd,
                     stride_d, alpha, beta, dtypes, epilogue=None, stride_bias=0, scales=None, stride_sfa=0,
                     stride_sfb=0, stream=None) -> int:
    """Direct call of the batched C entry point (arguments as for thl_gemm,
    plus the batch count and per-array strides in elements)."""
    opa = THL_OP_T if opA in ("T", THL_OP_T) else (THL_OP_N if opA in ("N", THL_OP_N) else int(opA))
    opb = THL_OP_T if opB in ("T", THL_OP_T) else (THL_OP_N if opB in ("N", THL_OP_N) else int(opB))
    return int(_lib.thl_gemm_batched(int(batch), int(m), int(n), int(k), A, int(lda), int(stride_a), opa, B,
                                     int(ldb), int(stride_b), opb, C, int(ldc), int(stride_c), D, int(ldd),
                                     int(stride_d), float(alpha), float(beta), ctypes.byref(dtypes),
                                     ctypes.byref(epilogue) if epilogue is not None else None, int(stride_bias),
                                     ctypes.byref(scales) if scales is not None else None, int(stride_sfa),
                                     int(stride_sfb), stream))


def thl_gemm_grouped(count, problems, problems_dev, opA, opB, alpha, beta, dtypes, epilogue=None, scales=None,
                     stream=None) -> int:
    """Direct call of the grouped C entry point: `problems` is a ctypes array
    of thl_group_problem (host), `problems_dev` the device address of a copy
    of the same bytes."""
    opa = THL_OP_T if opA in ("T", THL_OP_T) else THL_OP_N
    opb = THL_OP_T if opB in ("T", THL_OP_T) else THL_OP_N
    return int(_lib.thl_gemm_grouped(int(count), problems, problems_dev, opa, opb, float(alpha), float(beta),
                                     ctypes.byref(dtypes), ctypes.byref(epilogue) if epilogue is not None else None,
                                     ctypes.byref(scales) if scales is not None else None, stream))


def gemm(A, B, D, *, m, n, k, lda, ldb, ldd, op_a="T", op_b="N", C=None, ldc=0, alpha=1.0, beta=0.0,
         type_ab="bf16", type_c="f32", type_d="f32", bias=None, type_bias="none", act="none",
         a_scale=1.0, b_scale=1.0, sfa=None, ld_sfa=0, sfb=None, ld_sfb=0, stream=None, type_b=None,
         sfd=None, ld_sfd=0) -> str:
    """Torch-tensor convenience around thl_gemm: takes device tensors holding
    the stored bits, issues on the current stream, raises ThlError on a
    non-OK status and returns the name of the kernel variant launched.
    type_ab is A's format and B's unless type_b is given; sfd / ld_sfd take
    the generated scales of an MX-format D."""
    import torch

    def ptr(t):
        return None if t is None else t.data_ptr()

    flags = (THL_EPI_BIAS if bias is not None else 0) | {"none": 0, "relu": THL_EPI_RELU,
                                                         "gelu": THL_EPI_GELU}[act]
    epi = thl_epilogue(flags, ptr(bias), ptr(sfd), int(ld_sfd))
    sc = thl_scales(float(a_scale), float(b_scale), ptr(sfa), int(ld_sfa), ptr(sfb), int(ld_sfb))
    dts = make_dtypes(type_ab, type_b or type_ab, type_c, type_d, type_bias)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = thl_gemm(m, n, k, ptr(A), lda, op_a, ptr(B), ldb, op_b, ptr(C), ldc or max(1, m), ptr(D), ldd,
                  alpha, beta, dts, epi, sc, stream)
    if st != THL_OK:
        raise ThlError(st, "thl_gemm")
    return thl_last_variant()


def thl_kernel_index_map(name: str, points, params=()) -> list[tuple[int, int]]:
    """Evaluate a kernel index map at (x, y) points on the host."""
    pts = list(points)
    n = len(pts)
    arr_in = (ctypes.c_int64 * (2 * max(n, 1)))()
    for t, (x, y) in enumerate(pts):
        arr_in[2 * t], arr_in[2 * t + 1] = int(x), int(y)
    arr_out = (ctypes.c_int64 * (2 * max(n, 1)))()
    par = (ctypes.c_int64 * max(len(params), 1))(*[int(p) for p in params]) if params else None
    st = _lib.thl_kernel_index_map(name.encode(), par, n, arr_in, arr_out)
    if st != THL_OK:
        raise ThlError(st, f"thl_kernel_index_map({name})")
    return [(arr_out[2 * t], arr_out[2 * t + 1]) for t in range(n)]


def thl_kernel_index_map_names() -> list[str]:
    return _lib.thl_kernel_index_map_names().decode().split(",")


# ------------------------------------------------------------------ layouts

_CAP = 4096


def _text_call(fn, *args) -> str:
    buf = ctypes.create_string_buffer(_CAP)
    st = fn(*args, buf, _CAP)
    if st != THL_OK:
        raise ThlError(st, fn.__name__)
    return buf.value.decode()


def _enc(x) -> bytes:
    return x.encode() if isinstance(x, str) else x


def _tiler(t) -> bytes:
    return _enc(t if isinstance(t, str) else ";".join(t))


def thl_layout_coalesce(a: str) -> str:
    return _text_call(_lib.thl_layout_coalesce, _enc(a))


def thl_layout_composition(a: str, b) -> str:
    return _text_call(_lib.thl_layout_composition, _enc(a), _tiler(b))


def thl_layout_complement(a: str, cotarget: int) -> str:
    return _text_call(_lib.thl_layout_complement, _enc(a), int(cotarget))


def thl_layout_logical_divide(a: str, b) -> str:
    return _text_call(_lib.thl_layout_logical_divide, _enc(a), _tiler(b))


def thl_layout_zipped_divide(a: str, tiler) -> str:
    return _text_call(_lib.thl_layout_zipped_divide, _enc(a), _tiler(tiler))


def thl_layout_tiled_divide(a: str, tiler) -> str:
    return _text_call(_lib.thl_layout_tiled_divide, _enc(a), _tiler(tiler))


def thl_layout_flat_divide(a: str, tiler) -> str:
    return _text_call(_lib.thl_layout_flat_divide, _enc(a), _tiler(tiler))


def thl_layout_local_tile(a: str, tiler, tile: int) -> tuple[int, str]:
    off = ctypes.c_int64(0)
    s = _text_call(_lib.thl_layout_local_tile, _enc(a), _tiler(tiler), int(tile), ctypes.byref(off))
    return off.value, s


def thl_layout_local_partition(a: str, threads: str, tid: int) -> tuple[int, str]:
    off = ctypes.c_int64(0)
    s = _text_call(_lib.thl_layout_local_partition, _enc(a), _enc(threads), int(tid), ctypes.byref(off))
    return off.value, s


def thl_layout_eval(a: str, coords) -> list[int]:
    cs = [int(c) for c in coords]
    n = len(cs)
    arr = (ctypes.c_int64 * max(n, 1))(*cs)
    out = (ctypes.c_int64 * max(n, 1))()
    st = _lib.thl_layout_eval(_enc(a), arr, n, out)
    if st != THL_OK:
        raise ThlError(st, "thl_layout_eval")
    return list(out[:n])


def thl_layout_eval_coord(a: str, coord: str) -> int:
    out = ctypes.c_int64(0)
    st = _lib.thl_layout_eval_coord(_enc(a), _enc(coord), ctypes.byref(out))
    if st != THL_OK:
        raise ThlError(st, "thl_layout_eval_coord")
    return out.value


def thl_layout_info(a: str) -> tuple[int, int, int]:
    s, c, r = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    st = _lib.thl_layout_info(_enc(a), ctypes.byref(s), ctypes.byref(c), ctypes.byref(r))
    if st != THL_OK:
        raise ThlError(st, "thl_layout_info")
    return s.value, c.value, r.value


def thl_layout_mode(a: str, i: int) -> str:
    return _text_call(_lib.thl_layout_mode, _enc(a), int(i))


def thl_swizzle_eval(b: int, m: int, s: int, a: str, coords) -> list[int]:
    cs = [int(c) for c in coords]
    n = len(cs)
    arr = (ctypes.c_int64 * max(n, 1))(*cs)
    out = (ctypes.c_int64 * max(n, 1))()
    st = _lib.thl_swizzle_eval(int(b), int(m), int(s), _enc(a), arr, n, out)
    if st != THL_OK:
        raise ThlError(st, "thl_swizzle_eval")
    return list(out[:n])
