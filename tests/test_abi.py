"""The C-ABI library loads, exports every function include/thl.h declares,
and rejects bad problems before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import tile_hierarchy_linear_amd as thl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "thl.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(thl_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ("thl_gemm", "thl_status_string", "thl_last_variant", "thl_layout_coalesce",
                 "thl_layout_composition", "thl_layout_complement", "thl_layout_logical_divide",
                 "thl_layout_zipped_divide", "thl_layout_local_tile", "thl_layout_local_partition",
                 "thl_kernel_index_map"):
        assert must in names


@pytest.mark.parametrize("name", _declared_functions())
def test_every_declared_symbol_is_exported(name):
    lib = ctypes.CDLL(thl.LIB_PATH)
    assert hasattr(lib, name), name


def test_binding_names_match_the_c_entry_points():
    for name in _declared_functions():
        assert hasattr(thl, name), f"binding lacks {name}"


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert thl.thl_status_string(s)
    assert "unknown" in thl.thl_status_string(7)


def test_variants_are_listed():
    vs = thl.variants()
    assert len(vs) == thl.thl_variant_count() > 0
    for fam in ("bf16", "f16", "i8", "e4m3", "e5m2", "e2m1", "mxe4m3", "e4m3e5m2", "e5m2e4m3", "mxe5m2",
                "mxe4m3e5m2", "mxe5m2e4m3"):
        assert any(v.startswith(fam + "_") for v in vs)
    assert thl.thl_variant_name(-1) is None and thl.thl_variant_name(len(vs)) is None


# Fake (never dereferenced) device addresses, 256-byte aligned and far apart.
A, B, C, D, BIAS, SFA, SFB = (0x10000000 * i for i in range(1, 8))


def call(m=64, n=64, k=64, a=A, lda=None, opa="T", b=B, ldb=None, opb="N", c=None, ldc=None, d=D, ldd=None,
         alpha=1.0, beta=0.0, types=("bf16", "f32", "f32", "none"), flags=0, bias=None, sc=None, sfd=None,
         ld_sfd=0):
    ta, tc, td, tb = types
    lda = lda if lda is not None else max(1, k if opa == "T" else m)
    ldb = ldb if ldb is not None else max(1, k if opb == "N" else n)
    ldc = ldc if ldc is not None else max(1, m)
    ldd = ldd if ldd is not None else max(1, m)
    dts = thl.make_dtypes(ta, ta, tc, td, tb)
    epi = thl.thl_epilogue(flags, bias, sfd, ld_sfd)
    return thl.thl_gemm(m, n, k, a, lda, opa, b, ldb, opb, c, ldc, d, ldd, alpha, beta, dts, epi, sc, None)


def test_negative_dimensions():
    assert call(m=-1) == thl.THL_ERR_INVALID
    assert call(k=-5) == thl.THL_ERR_INVALID


def test_bound_call_validates_like_the_direct_call():
    # bind_thl_gemm marshals once and repeats the same call: same statuses as thl_gemm
    dts, epi = thl.make_dtypes("bf16", "bf16", "f32", "f32"), thl.thl_epilogue(0, None, None, 0)
    for entry in ("thl_gemm", "thl_gemm_noalloc"):
        bad_m = thl.bind_thl_gemm(-1, 64, 64, A, 64, "T", B, 64, "N", None, 64, D, 64, 1.0, 0.0, dts, epi, None,
                                  None, entry)
        assert bad_m() == bad_m() == thl.THL_ERR_INVALID
        bad_ld = thl.bind_thl_gemm(64, 64, 64, A, 63, "T", B, 64, "N", None, 64, D, 64, 1.0, 0.0, dts, epi, None,
                                   None, entry)
        assert bad_ld() == thl.THL_ERR_INVALID
    assert call(lda=63) == thl.THL_ERR_INVALID


def test_leading_dimension_too_small():
    assert call(lda=63) == thl.THL_ERR_INVALID
    assert call(ldb=10) == thl.THL_ERR_INVALID
    assert call(ldd=32) == thl.THL_ERR_INVALID
    assert call(beta=1.0, c=C, ldc=8) == thl.THL_ERR_INVALID


def test_null_pointers():
    assert call(d=None) == thl.THL_ERR_INVALID
    assert call(a=None) == thl.THL_ERR_INVALID
    assert call(beta=1.0, c=None) == thl.THL_ERR_INVALID
    assert call(flags=thl.THL_EPI_BIAS, bias=None, types=("bf16", "f32", "f32", "f32")) == thl.THL_ERR_INVALID


def test_bad_flags_and_ops():
    assert call(flags=thl.THL_EPI_RELU | thl.THL_EPI_GELU) == thl.THL_ERR_INVALID
    assert call(flags=64) == thl.THL_ERR_INVALID
    assert call(opa=7) == thl.THL_ERR_INVALID


def test_unsupported_combinations():
    assert call(types=("f32", "f32", "f32", "none")) == thl.THL_ERR_UNSUPPORTED  # fp32 operands
    dts = thl.make_dtypes("bf16", "f16", "f32", "f32")
    assert thl.thl_gemm(64, 64, 64, A, 64, "T", B, 64, "N", None, 64, D, 64, 1.0, 0.0, dts, None, None,
                        None) == thl.THL_ERR_UNSUPPORTED
    assert call(types=("i8", "f32", "f32", "none")) == thl.THL_ERR_UNSUPPORTED  # int8 needs int32 out
    assert call(types=("i8", "i32", "i32", "none"), alpha=2.0) == thl.THL_ERR_UNSUPPORTED
    assert call(types=("i8", "i32", "i32", "none"), beta=0.5, c=C) == thl.THL_ERR_UNSUPPORTED
    sc = thl.thl_scales(1.0, 1.0, SFA, 1, SFB, 1)
    assert call(types=("e2m1", "f32", "bf16", "none"), k=48, sc=sc) == thl.THL_ERR_UNSUPPORTED  # k % 32
    mixed = thl.make_dtypes("e4m3", "bf16", "f32", "bf16")  # mixed only within fp8
    assert thl.thl_gemm(64, 64, 64, A, 64, "T", B, 64, "N", None, 64, D, 64, 1.0, 0.0, mixed, None, None,
                        None) == thl.THL_ERR_UNSUPPORTED
    mixed8 = thl.make_dtypes("e4m3", "e5m2", "f32", "bf16")
    assert thl.thl_gemm(64, 0, 64, A, 64, "T", B, 64, "N", None, 64, D, 64, 1.0, 0.0, mixed8, None, None,
                        None) == thl.THL_OK
    assert thl.thl_last_variant().startswith("e4m3e5m2_")


@pytest.mark.parametrize("fmt,td", [("bf16", "f32"), ("f16", "f32"), ("i8", "i32")])
def test_block_scales_with_formats_that_take_none_are_refused(fmt, td):
    # A block-scale array given with a format that has no block-scaled kernel
    # is refused, not dropped (the result would ignore the caller's scales).
    tc = "i32" if fmt == "i8" else "f32"
    for sc in (thl.thl_scales(1.0, 1.0, SFA, 16, SFB, 16), thl.thl_scales(1.0, 1.0, SFA, 16, None, 0),
               thl.thl_scales(1.0, 1.0, None, 0, SFB, 16)):
        assert call(types=(fmt, tc, td, "none"), sc=sc) == thl.THL_ERR_UNSUPPORTED
        assert call(m=0, types=(fmt, tc, td, "none"), sc=sc) == thl.THL_ERR_UNSUPPORTED


@pytest.mark.parametrize("fa,fb,mx,plain", [("e4m3", "e4m3", "mxe4m3_", "e4m3_"), ("e5m2", "e5m2", "mxe5m2_", "e5m2_"),
                                             ("e4m3", "e5m2", "mxe4m3e5m2_", "e4m3e5m2_"),
                                             ("e5m2", "e4m3", "mxe5m2e4m3_", "e5m2e4m3_")])
def test_fp8_block_scales_both_or_neither(fa, fb, mx, plain):
    # fp8 operands with scale arrays are MX fp8 (one scale per 32 K-elements),
    # with neither plain fp8; one alone is an error when there is work to do.
    dts = thl.make_dtypes(fa, fb, "f32", "bf16")

    def go(sc, m=64):
        return thl.thl_gemm(m, 64, 64, A, 64, "T", B, 64, "N", None, 64, D, 64, 1.0, 0.0, dts, None, sc, None)

    for sc in (thl.thl_scales(1.0, 1.0, SFA, 16, None, 0), thl.thl_scales(1.0, 1.0, None, 0, SFB, 16)):
        assert go(sc) == thl.THL_ERR_INVALID
        # with no outputs nothing is read: one array (for the non-empty operand) is enough
        assert go(sc, m=0) == thl.THL_OK
        assert thl.thl_last_variant().startswith(mx)
    assert go(thl.thl_scales(1.0, 1.0, SFA, 16, SFB, 16), m=0) == thl.THL_OK
    assert thl.thl_last_variant().startswith(mx)
    assert go(None, m=0) == thl.THL_OK
    assert thl.thl_last_variant().startswith(plain)


def test_mxfp4_needs_both_scale_arrays():
    # one array without the other is refused; none at all is plain fp4 (run
    # by way of the conversion pass, so only the quick return works here)
    assert call(types=("e2m1", "f32", "bf16", "none"), sc=thl.thl_scales(1.0, 1.0, SFA, 16, None, 0)) == \
        thl.THL_ERR_INVALID
    assert call(types=("e2m1", "f32", "bf16", "none"), sc=None, m=0) == thl.THL_OK
    assert thl.thl_last_variant().endswith("+cvt_ab")
    sc = thl.thl_scales(1.0, 1.0, SFA, 1, SFB, 2)  # ld_sfa < k/32
    assert call(types=("e2m1", "f32", "bf16", "none"), sc=sc) == thl.THL_ERR_INVALID
    sc = thl.thl_scales(1.0, 1.0, SFA, 4, SFB, 4)
    assert call(types=("e2m1", "f32", "bf16", "none"), lda=65, sc=sc) == thl.THL_ERR_INVALID  # odd ld


def test_mxfp4_scale_rows_must_be_16_byte_aligned():
    sc = thl.thl_scales(1.0, 1.0, SFA, 4, SFB, 16)  # ld_sfa = 4: not a multiple of 16
    assert call(types=("e2m1", "f32", "bf16", "none"), sc=sc) == thl.THL_ERR_MISALIGNED
    sc = thl.thl_scales(1.0, 1.0, SFA + 4, 16, SFB, 16)
    assert call(types=("e2m1", "f32", "bf16", "none"), sc=sc) == thl.THL_ERR_MISALIGNED
    sc = thl.thl_scales(1.0, 1.0, SFA, 16, SFB, 16)  # accepted (the launch itself needs a GPU)
    assert call(types=("e2m1", "f32", "bf16", "none"), sc=sc) in (thl.THL_OK, thl.THL_ERR_HIP)


def test_misaligned_16bit_lines_take_the_pass():
    # bf16 rows of 63 elements = 126 bytes, or a base 2 bytes off, fit no
    # kernel: the pass re-pitches them in their own layout (m = 0 runs the
    # choice and validation without touching a device)
    assert call(m=0, k=63, lda=63, ldb=64) == thl.THL_OK
    assert thl.thl_last_variant().endswith("+cvt_a") and "_tn_" in thl.thl_last_variant()
    assert call(m=0, a=A + 2) == thl.THL_OK
    assert thl.thl_last_variant().endswith("+cvt_a")
    assert call(m=0, opa="N", lda=8, opb="T", ldb=65) == thl.THL_OK
    assert thl.thl_last_variant().endswith("+cvt_b") and "_nt_" in thl.thl_last_variant()
    # 4-byte lines that are not 16-byte units stay on the 4-byte-copy kernels
    assert call(m=0, k=64, lda=66, ldb=64) == thl.THL_OK
    assert "+cvt" not in thl.thl_last_variant() and "_v4_" in thl.thl_last_variant()
    # a forced variant keeps the caller's lines, which it cannot read
    os.environ["THL_FORCE_VARIANT"] = "bf16_tn_128x128_v4_s4_o2"
    try:
        assert call(m=0, k=63, lda=63, ldb=64) == thl.THL_ERR_UNSUPPORTED
    finally:
        del os.environ["THL_FORCE_VARIANT"]


def test_overlaps():
    # D over A
    assert call(d=A) == thl.THL_ERR_INVALID
    assert call(d=B + 64) == thl.THL_ERR_INVALID
    # partial overlap with C
    assert call(beta=1.0, c=C, d=C + 4) == thl.THL_ERR_INVALID
    # bias overlapping D
    assert call(flags=thl.THL_EPI_BIAS, bias=D + 8, types=("bf16", "f32", "f32", "f32")) == thl.THL_ERR_INVALID


def test_quick_returns_do_not_launch():
    # m == 0 or n == 0: OK without touching the device (works without a GPU)
    assert call(m=0) == thl.THL_OK
    assert call(n=0) == thl.THL_OK
    assert call(m=0, n=0, k=0, a=None, b=None, d=None) == thl.THL_OK


def test_forced_variant_must_fit():
    os.environ["THL_FORCE_VARIANT"] = "i8_tn_256x256_v16_s4_o1"
    try:
        assert call(m=0) == thl.THL_ERR_UNSUPPORTED  # bf16 problem, int8 variant
    finally:
        del os.environ["THL_FORCE_VARIANT"]


@pytest.mark.parametrize("fam,ta,td", [("bf16", "bf16", "bf16"), ("f16", "f16", "f32"), ("i8", "i8", "i32"),
                                       ("e4m3", "e4m3", "bf16"), ("e5m2", "e5m2", "bf16"),
                                       ("e2m1", "e2m1", "bf16")])
def test_small_m_selection(fam, ta, td):
    # n == 0 selects a variant without a launch (no GPU needed)
    tc = "i32" if ta == "i8" else "f32"
    types = (ta, tc, td, "none")
    k = 8192
    # MXFP4 with its block scales (E2M1 without them is plain fp4, run by way of fp8)
    sc = thl.thl_scales(1.0, 1.0, SFA, 256, SFB, 256) if ta == "e2m1" else None

    def go(**kw):
        return call(sc=sc, **kw)

    for m, rows in ((1, 16), (7, 16), (16, 16), (17, 32), (32, 32), (33, 64), (64, 64)):
        assert go(m=m, n=0, k=k, types=types) == thl.THL_OK
        assert thl.thl_last_variant() == f"{fam}_tn_skinny{rows}_k4"
    assert go(m=65, n=0, k=k, types=types) == thl.THL_OK
    assert "skinny" not in thl.thl_last_variant()
    # k == 0, or operands that are not 16-byte units: the tiled kernels
    assert go(m=1, n=0, k=0, lda=64, ldb=64, types=types) == thl.THL_OK
    assert "skinny" not in thl.thl_last_variant()
    assert go(m=1, n=0, k=k, a=A + 4, types=types) == thl.THL_OK
    assert "skinny" not in thl.thl_last_variant()
    if fam in ("bf16", "f16"):  # M-major A: the tiled kernels
        assert go(m=1, n=0, k=k, opa="N", lda=8, types=types) == thl.THL_OK
        assert "skinny" not in thl.thl_last_variant()
    # forcing a small-M variant on more rows than it covers is refused
    for rows in (16, 64):
        os.environ["THL_FORCE_VARIANT"] = f"{fam}_tn_skinny{rows}_k4"
        try:
            assert go(m=rows, n=0, k=k, types=types) == thl.THL_OK
            assert go(m=rows + 1, n=0, k=k, types=types) == thl.THL_ERR_UNSUPPORTED
        finally:
            del os.environ["THL_FORCE_VARIANT"]


def bcall(batch=2, m=64, n=64, k=64, sa=None, sb=None, sc=0, sd=None, sbias=0, d=D, c=None, beta=0.0,
          types=("bf16", "f32", "f32", "none"), lda=None, ldb=None, opa="T", opb="N", a=A, b=B, bias=None,
          flags=0, sc_struct=None, ssfa=0, ssfb=0):
    ta, tc, td, tb = types
    lda = lda if lda is not None else max(1, k if opa == "T" else m)
    ldb = ldb if ldb is not None else max(1, k if opb == "N" else n)
    sa = sa if sa is not None else lda * (m if opa == "T" else k)
    sb = sb if sb is not None else ldb * (n if opb == "N" else k)
    sd = sd if sd is not None else m * n
    dts = thl.make_dtypes(ta, ta, tc, td, tb)
    epi = thl.thl_epilogue(flags, bias)
    return thl.thl_gemm_batched(batch, m, n, k, a, lda, sa, opa, b, ldb, sb, opb, c, max(1, m), sc, d, max(1, m), sd,
                                1.0, beta, dts, epi, sbias, sc_struct, ssfa, ssfb, None)


def test_huge_leading_dimensions_and_strides_are_refused():
    # spans are computed in int64: ld above INT32_MAX and batch strides
    # above 2^40 are refused before any arithmetic could overflow
    assert call(ldd=2 ** 31) == thl.THL_ERR_UNSUPPORTED
    assert call(c=C, beta=1.0, ldc=2 ** 40) == thl.THL_ERR_UNSUPPORTED
    assert bcall(sd=2 ** 41) == thl.THL_ERR_UNSUPPORTED
    assert bcall(sa=2 ** 62) == thl.THL_ERR_UNSUPPORTED


def test_batched_validation():
    # batch 0 and empty problems return at once (no GPU needed)
    assert bcall(batch=0) == thl.THL_OK
    assert bcall(n=0) == thl.THL_OK
    assert bcall(batch=-1) == thl.THL_ERR_INVALID
    assert bcall(batch=65536) == thl.THL_ERR_UNSUPPORTED
    for kw in ({"sa": -1}, {"sb": -64}, {"sd": -4096}, {"sbias": -1}):
        assert bcall(**kw) == thl.THL_ERR_INVALID
    # D matrices of two problems overlap
    assert bcall(sd=64 * 64 - 1) == thl.THL_ERR_INVALID
    assert bcall(sd=0) == thl.THL_ERR_INVALID
    # D's span over the batch reaches A's span (A right after the first D)
    assert bcall(a=D + 4 * 64 * 64, sd=2 * 64 * 64) == thl.THL_ERR_INVALID
    # C may alias D only with the same stride
    assert bcall(c=D, beta=1.0, sc=64 * 64 + 64, types=("bf16", "f32", "f32", "none")) == thl.THL_ERR_INVALID
    # fp4 operand strides count fp4 elements and must be even
    assert bcall(sa=33, k=64, types=("e2m1", "bf16", "bf16", "none"), lda=64, ldb=64) == thl.THL_ERR_INVALID
    # a stride that breaks every variant's 4-byte alignment (the second
    # problem's A would start 2 bytes off): re-pitched by the pass
    assert bcall(n=0, sa=64 * 64 + 1) == thl.THL_OK  # selection runs before the quick return
    assert thl.thl_last_variant().endswith("+cvt_a")


# ------------------------------------------------------------ grouped problems

def _gp(m=64, n=64, k=64, a=A, lda=None, b=B, ldb=None, c=None, ldc=None, d=D, ldd=None, bias=None, sfa=None,
        ld_sfa=0, sfb=None, ld_sfb=0):
    return thl.thl_group_problem(m, n, k, a, lda if lda is not None else max(1, k), b,
                                 ldb if ldb is not None else max(1, k), c, ldc if ldc is not None else max(1, m), d,
                                 ldd if ldd is not None else max(1, m), bias, sfa, ld_sfa, sfb, ld_sfb)


def gcall(problems, dev=0x70000000, opa="T", opb="N", alpha=1.0, beta=0.0, types=("bf16", "f32", "f32", "none"),
          flags=0, sc=None):
    ta, tc, td, tb = types
    arr = (thl.thl_group_problem * max(1, len(problems)))(*problems)
    dts = thl.make_dtypes(ta, ta, tc, td, tb)
    return thl.thl_gemm_grouped(len(problems), arr, dev, opa, opb, alpha, beta, dts, thl.thl_epilogue(flags, None),
                                sc, None)


def test_grouped_validation():
    assert gcall([]) == thl.THL_OK
    dts = thl.make_dtypes("bf16", "bf16", "f32", "f32")
    assert thl.thl_gemm_grouped(-1, None, None, "T", "N", 1.0, 0.0, dts, None, None, None) == thl.THL_ERR_INVALID
    assert thl.thl_gemm_grouped(2, None, None, "T", "N", 1.0, 0.0, dts, None, None, None) == thl.THL_ERR_INVALID
    assert thl.thl_gemm_grouped(70000, None, None, "T", "N", 1.0, 0.0, dts, None, None, None) == \
        thl.THL_ERR_UNSUPPORTED
    # one bad problem fails the group
    assert gcall([_gp(), _gp(lda=10, d=D + 0x100000)]) == thl.THL_ERR_INVALID
    # no launch when no problem has outputs; the variant is still chosen
    assert gcall([_gp(m=0), _gp(n=0, d=D + 0x100000)]) == thl.THL_OK
    assert thl.thl_last_variant().startswith("bf16_tn_")
    # work to do needs the device copy of the descriptors
    assert gcall([_gp()], dev=None) == thl.THL_ERR_INVALID
    # accepted (the launch itself needs a GPU)
    assert gcall([_gp(), _gp(m=100, n=37, d=D + 0x100000)]) in (thl.THL_OK, thl.THL_ERR_HIP)


def test_grouped_outputs_may_not_overlap_across_problems():
    # D of problem 1 inside D of problem 0
    assert gcall([_gp(), _gp(d=D + 64)]) == thl.THL_ERR_INVALID
    # D of problem 1 over A of problem 0
    assert gcall([_gp(), _gp(d=A)]) == thl.THL_ERR_INVALID
    # D of problem 0 over problem 1's C (beta != 0)
    assert gcall([_gp(c=C), _gp(c=D, d=D + 0x100000)], beta=1.0) == thl.THL_ERR_INVALID
    # each problem may read its own C in place (C == D), and problems may share inputs
    assert gcall([_gp(c=D), _gp(c=D + 0x100000, d=D + 0x100000)], beta=1.0) in (thl.THL_OK, thl.THL_ERR_HIP)


def test_grouped_needs_one_family():
    # fp8 problems with block scales and without them would be two families
    sc = [_gp(sfa=SFA, ld_sfa=16, sfb=SFB, ld_sfb=16), _gp(d=D + 0x100000)]
    assert gcall(sc, types=("e4m3", "f32", "bf16", "none")) == thl.THL_ERR_INVALID
    assert gcall([sc[0], _gp(d=D + 0x100000, sfa=SFA, ld_sfa=16, sfb=SFB + 0x10000, ld_sfb=16)],
                 types=("e4m3", "f32", "bf16", "none")) in (thl.THL_OK, thl.THL_ERR_HIP)


# ------------------------------------------------------------ MX-format D

SFD = 0x80000000


@pytest.mark.parametrize("td", ["e2m1", "e4m3", "e5m2"])
def test_mx_output_needs_its_scale_array(td):
    mx = dict(types=("bf16", "f32", td, "none"), ldd=64)
    assert call(**mx) == thl.THL_ERR_INVALID                       # no scale array
    assert call(m=100, ldd=100, sfd=SFD, ld_sfd=3, types=mx["types"]) == thl.THL_ERR_INVALID  # < ceil(100/32)
    # no rows or no columns: nothing is written, no scale array needed;
    # the selection still names an MX-output variant
    assert call(m=0, **mx) == thl.THL_OK
    assert thl.thl_last_variant().endswith("_mxout")
    assert call(n=0, **mx) == thl.THL_OK


def test_mx_output_e2m1_column_starts_on_whole_bytes():
    # two E2M1 codes a byte along M: an odd ldd would start every other column mid-byte
    assert call(m=63, ldd=63, sfd=SFD, ld_sfd=2, types=("bf16", "f32", "e2m1", "none")) == thl.THL_ERR_INVALID


def test_mx_output_scales_overlap_nothing():
    types = ("bf16", "f32", "e4m3", "none")
    # D spans 64 x 64 bytes from D; scales 2 x 64 bytes
    assert call(sfd=D + 64 * 63, ld_sfd=2, types=types) == thl.THL_ERR_INVALID
    assert call(sfd=A + 16, ld_sfd=2, types=types) == thl.THL_ERR_INVALID
    assert call(sfd=BIAS, ld_sfd=2, bias=BIAS + 8, flags=thl.THL_EPI_BIAS, types=("bf16", "f32", "e4m3", "f32")) \
        == thl.THL_ERR_INVALID


def test_mx_output_is_for_single_float_problems():
    types = ("bf16", "f32", "e4m3", "none")
    assert bcall(types=types, sd=64 * 64) == thl.THL_ERR_UNSUPPORTED
    assert gcall([_gp()], types=types) == thl.THL_ERR_UNSUPPORTED
    # integer GEMMs write int32
    assert call(types=("i8", "i32", "e4m3", "none"), sfd=SFD, ld_sfd=2) == thl.THL_ERR_UNSUPPORTED


def test_mx_output_re_pitches_operand_lines_off_16_byte_units():
    # bf16 B lines of 130 elements (260 bytes): the MX-output kernels load
    # 16-byte units only, so the pass re-pitches them (m = 0: choice and
    # validation only)
    types = ("bf16", "f32", "e4m3", "none")
    assert call(n=130, opb="T", ldb=130, sfd=SFD, ld_sfd=2, types=types, m=0) == thl.THL_OK
    assert thl.thl_last_variant().endswith("_mxout+cvt_b"), thl.thl_last_variant()
    assert call(n=130, opb="T", ldb=136, sfd=SFD, ld_sfd=2, types=types, m=0) == thl.THL_OK
    assert "+cvt" not in thl.thl_last_variant()
    # fp8 rows of 68 bytes: the same
    assert call(types=("e4m3", "f32", "e4m3", "none"), k=64, lda=68, ldb=64, sfd=SFD, ld_sfd=2, m=0) == thl.THL_OK
    assert thl.thl_last_variant().endswith("_mxout+cvt_a"), thl.thl_last_variant()


# ------------------------------------------------------------ the conversion pass

@pytest.mark.parametrize("types,ops,which", [
    (("i8", "i32", "i32", "none"), ("N", "N"), "a"),
    (("e4m3", "f32", "bf16", "none"), ("T", "T"), "b"),
    (("e5m2", "f32", "bf16", "none"), ("N", "T"), "ab"),
    (("e2m3", "f32", "bf16", "none"), ("T", "N"), "ab"),
    (("e3m2", "f32", "bf16", "none"), ("N", "N"), "ab"),
])
def test_layouts_and_formats_the_tiles_cannot_stage_take_the_pass(types, ops, which):
    # m = 0: the quick return still picks the K-major run and names the pass
    assert call(m=0, types=types, opa=ops[0], opb=ops[1], lda=64, ldb=64) == thl.THL_OK
    v = thl.thl_last_variant()
    assert v.endswith("+cvt_" + which), v
    inner = {"i8": "i8_", "e4m3": "e4m3_", "e5m2": "e5m2_", "e2m3": "e4m3_", "e3m2": "e4m3_"}[types[0]]
    assert v.startswith(inner) and "_tn_" in v, v


def test_conversion_pass_validation():
    f6 = ("e2m3", "f32", "bf16", "none")
    # fp6 lines start on whole bytes: leading dimensions a multiple of 4 elements
    assert call(types=f6, lda=66) == thl.THL_ERR_INVALID
    assert call(types=f6, opa="N", lda=66) == thl.THL_ERR_INVALID
    # block-scaled fp6: k % 32 and both scale arrays, as for the other MX formats
    assert call(types=f6, k=48, sc=thl.thl_scales(1.0, 1.0, SFA, 16, SFB, 16)) == thl.THL_ERR_UNSUPPORTED
    assert call(types=f6, sc=thl.thl_scales(1.0, 1.0, SFA, 16, None, 0)) == thl.THL_ERR_INVALID
    # fp6 beside a 16-bit operand: no path
    dts = thl.make_dtypes("e2m3", "bf16", "f32", "bf16")
    assert thl.thl_gemm(64, 64, 64, A, 64, "T", B, 64, "N", None, 64, D, 64, 1.0, 0.0, dts, None, None,
                        None) == thl.THL_ERR_UNSUPPORTED
    # D overlapping the caller's operand stored along M
    assert call(types=("e4m3", "f32", "bf16", "none"), opa="N", d=A + 64) == thl.THL_ERR_INVALID
    # the K-major run's own rules (int8: alpha 1) are checked before anything runs
    assert call(types=("i8", "i32", "i32", "none"), opa="N", alpha=2.0) == thl.THL_ERR_UNSUPPORTED


def test_no_alloc_entry_point_bounds_the_converted_operands():
    # two 8192 x 8192 fp8 operands rewritten: 128 MiB, past the 40 MiB scratch;
    # refused before any device call
    dts = thl.make_dtypes("e4m3", "e4m3", "f32", "bf16")
    assert thl.thl_gemm_noalloc(8192, 8192, 8192, A, 8192, "N", B, 8192, "T", None, 8192, D, 8192, 1.0, 0.0, dts,
                                None, None, None) == thl.THL_ERR_SCRATCH


def test_rows_off_every_kernel_alignment_take_the_pass():
    # fp8 rows of 2041 bytes fit no kernel (they need 4-byte units): rewritten
    # whatever the size; bf16 rows of odd length are re-pitched as bf16
    assert call(m=0, types=("e4m3", "f32", "bf16", "none"), k=2041, lda=2041, ldb=2041) == thl.THL_OK
    assert thl.thl_last_variant().endswith("+cvt_ab")
    assert call(m=0, types=("e4m3", "f32", "bf16", "none"), k=2040, lda=2040, ldb=2040) == thl.THL_OK
    assert "+cvt" not in thl.thl_last_variant() and "_v4_" in thl.thl_last_variant()
    assert call(m=0, types=("bf16", "f32", "f32", "none"), k=63, lda=63, ldb=63) == thl.THL_OK
    assert thl.thl_last_variant().endswith("+cvt_ab")

