"""Pins for the parity comparison (oracle/compare.py): the tolerance and the
dequantized operand maxima it is built from.

The float bar is 2^-20 * K * |alpha| * max|a'| * max|b'| * g + ulp_out(y), with
a', b' the dequantized operands (per-tensor scales for fp8, one E8M0 scale
per 32 K-elements for the MX formats) and g = 1.13 for GELU.  Every expected
number below is worked out by hand from the stored codes, so a mistake in how
the maxima are taken (a scale dropped or applied twice, blocks scaled by the
wrong exponent, padding read as data) or in the bound's terms fails a test.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import compare


def _w(**kw):
    base = dict(name="hand", m=1, n=1, k=32, type_a="f16", type_b="f16", type_d="f32", op_a="T", op_b="N",
                lda=32, ldb=32, ldd=1, a=np.zeros((1, 32), np.uint16), b=np.zeros((1, 32), np.uint16))
    base.update(kw)
    return wl.Workload(**base)


# ------------------------------------------------------------- float_tolerance

def test_tolerance_terms_by_hand():
    # 2^-20 * 64 * |-2| * 3 * 5 = 1920 * 2^-20; fp32 ulp at 1.0 is 2^-23
    tol = compare.float_tolerance(64, -2.0, 3.0, 5.0, "f32", np.array([1.0]))
    assert tol[0] == 1920 * 2.0 ** -20 + 2.0 ** -23


def test_tolerance_gelu_factor():
    tol = compare.float_tolerance(64, 1.0, 1.0, 1.0, "f32", np.array([0.0]), act="gelu")
    assert tol[0] == 64 * 2.0 ** -20 * 1.13 + 2.0 ** -149


def test_tolerance_relu_has_no_factor():
    tol = compare.float_tolerance(64, 1.0, 1.0, 1.0, "bf16", np.array([0.0]), act="relu")
    assert tol[0] == 64 * 2.0 ** -20 + 2.0 ** -133


@pytest.mark.parametrize("fmt,y,ulp", [
    ("bf16", 3.0, 2.0 ** -6),      # 3 = 1.5 * 2^1, 8 significant bits
    ("bf16", -3.0, 2.0 ** -6),
    ("bf16", 1.0, 2.0 ** -7),
    ("bf16", 0.99, 2.0 ** -8),
    ("f16", 1024.0, 1.0),
    ("f16", 0.0, 2.0 ** -24),      # subnormal spacing at zero
    ("f16", 2.0 ** -20, 2.0 ** -24),
    ("f32", 2.0 ** 24, 2.0),
])
def test_tolerance_ulp_term_alone(fmt, y, ulp):
    assert compare.float_tolerance(0, 1.0, 7.0, 7.0, fmt, np.array([y]))[0] == ulp


# ------------------------------------------------------------- operand maxima

def test_operand_max_plain_formats():
    a = wl.encode(np.array([[0.5, -3.0, 2.0]]), "f16")
    b = wl.encode(np.array([[1.0, 0.25, -0.75]]), "f16")
    w = _w(k=3, lda=3, ldb=3, a=a, b=b)
    assert compare.operand_max_abs(w, "a") == 3.0
    assert compare.operand_max_abs(w, "b") == 1.0


def test_operand_max_per_tensor_fp8():
    # e4m3 0xFE = -448, a_scale 1/4 -> 112;  e5m2 0x7B = 57344, b_scale 2^-10 -> 56
    a = np.array([[0x38, 0xFE, 0x01, 0x40]], np.uint8)
    b = np.array([[0x7B, 0x3C, 0x80, 0x01]], np.uint8)
    w = _w(k=4, lda=4, ldb=4, type_a="e4m3", type_b="e5m2", a=a, b=b, a_scale=0.25, b_scale=2.0 ** -10)
    assert compare.operand_max_abs(w, "a") == 112.0
    assert compare.operand_max_abs(w, "b") == 56.0


def _mx_scales(rows, blocks, pad_code):
    sf = np.full((rows, 16), pad_code, np.uint8)
    for r, row in enumerate(blocks):
        sf[r, : len(row)] = row
    return sf


def test_operand_max_mxfp8_blockwise():
    # A: 2 rows x 64 K (two blocks), e4m3 codes; per-tensor a_scale 1/2.
    #   row 0: block 0 max 448 (0x7E) at scale 2^-3 -> 56; block 1 max 2 (0x40) at 2^4 -> 32
    #   row 1: block 0 max 1 (0x38) at 2^6 -> 64; block 1 zero at 2^9
    #   -> max |a'| = 64 * 1/2 = 32.  The naive max|q| * max scale would be 448 * 2^9.
    # Byte 64 of each row is padding past K (0x7E) and scale bytes past K/32 are
    # 0xFF (the E8M0 NaN): neither may count.
    a = np.zeros((2, 80), np.uint8)
    a[0, 3], a[0, 40], a[1, 5] = 0x7E, 0x40, 0x38
    a[:, 64:] = 0x7E
    sfa = _mx_scales(2, [[124, 131], [133, 136]], 0xFF)
    # B: 1 row, block 0 max 0.5 (0x30) at 2^2 -> 2, block 1 max 448 at 2^-8 -> 1.75
    b = np.zeros((1, 64), np.uint8)
    b[0, 0], b[0, 33] = 0x30, 0x7E
    sfb = _mx_scales(1, [[129, 119]], 0xFF)
    w = _w(m=2, n=1, k=64, lda=80, ldb=64, type_a="e4m3", type_b="e4m3", a=a, b=b, sfa=sfa, ld_sfa=16,
           sfb=sfb, ld_sfb=16, a_scale=0.5, b_scale=1.0)
    assert compare.operand_max_abs(w, "a") == 32.0
    assert compare.operand_max_abs(w, "b") == 2.0


def test_operand_max_mxfp4_blockwise():
    # A: 1 row x 64 K of e2m1 codes.  Block 0 holds -6 (code 0xF) at scale 2^-2
    # -> 1.5; block 1 holds 0.5 (code 0x1) at 2^3 -> 4.  max |a'| = 4 (the
    # largest raw code, 6, sits in the block with the smaller scale).
    codes = np.zeros((1, 64), np.uint8)
    codes[0, 7], codes[0, 50] = 0xF, 0x1
    a = wl.pack_e2m1(codes)
    sfa = _mx_scales(1, [[125, 130]], 0xFF)
    # B: block 0 holds 4 (0x6) at 2^5 -> 128; block 1 holds 6 at 2^0 -> 6
    cb = np.zeros((1, 64), np.uint8)
    cb[0, 1], cb[0, 63] = 0x6, 0x7
    b = wl.pack_e2m1(cb)
    sfb = _mx_scales(1, [[132, 127]], 0xFF)
    w = _w(k=64, lda=64, ldb=64, type_a="e2m1", type_b="e2m1", a=a, b=b, sfa=sfa, ld_sfa=16, sfb=sfb,
           ld_sfb=16)
    assert compare.operand_max_abs(w, "a") == 4.0
    assert compare.operand_max_abs(w, "b") == 128.0


# ------------------------------------------------------------- the check itself

def test_parity_check_accepts_inside_and_rejects_outside_the_bar():
    # 1 x 1 x 32 f16 GEMM, A = B = 1: y = 32, fp32 out.  Bar = 32 * 2^-20 + 2^-18.
    a = wl.encode(np.ones((1, 32)), "f16")
    w = _w(a=a, b=a.copy())
    bar = 32 * 2.0 ** -20 + 2.0 ** -18
    rows, cols = np.array([0]), np.array([0])
    assert compare.parity_check(w, np.array([32.0 + 0.99 * bar]), rows, cols)["ok"]
    assert not compare.parity_check(w, np.array([32.0 + 1.01 * bar]), rows, cols)["ok"]
    assert not compare.parity_check(w, np.array([np.nan]), rows, cols)["ok"]


def test_exact_check_for_integers():
    assert compare.check_exact(np.array([3, -4]), np.array([3, -4]))["ok"]
    r = compare.check_exact(np.array([3, -4]), np.array([3, -5]))
    assert not r["ok"] and r["n_bad"] == 1


def test_operand_max_mx_e5m2_keeps_the_per_tensor_scale():
    # MX fp8 with E5M2 elements: 0x7B = 57344 at block scale 2^-10 -> 56, times
    # the per-tensor scale 1/4 -> 14 (the per-tensor scales multiply every fp8
    # family, block-scaled or not)
    a = np.zeros((1, 32), np.uint8)
    a[0, 9] = 0x7B
    sfa = _mx_scales(1, [[117]], 0xFF)
    w = _w(k=32, lda=32, ldb=32, type_a="e5m2", type_b="e5m2", a=a, b=a.copy(), sfa=sfa, ld_sfa=16,
           sfb=sfa.copy(), ld_sfb=16, a_scale=0.25, b_scale=1.0)
    assert compare.operand_max_abs(w, "a") == 14.0
    assert compare.operand_max_abs(w, "b") == 56.0


def test_operand_max_m_major_block_scaled():
    # A stored along M (op N): 64 k-lines of lda = 2 e4m3 codes.  A(0, 5) = 448
    # (0x7E) at SFA(0, 0) = 2^-3 -> 56; A(1, 40) = 2 (0x40) at SFA(1, 1) = 2^4
    # -> 32; A(0, 40) = 1 (0x38) at SFA(0, 1) = 2^-8.  max |a'| = 56.  Read as
    # K-major rows (the wrong way) the same bytes give 448 * 2^-3 in no place
    # and 2 at scale 2^4 in row 0 (32), so the maximum would differ.
    a = np.zeros((64, 2), np.uint8)
    a[5, 0], a[40, 1], a[40, 0] = 0x7E, 0x40, 0x38
    sfa = _mx_scales(2, [[124, 119], [127, 131]], 0xFF)
    b = np.zeros((1, 64), np.uint8)
    b[0, 0] = 0x38
    sfb = _mx_scales(1, [[127, 127]], 0xFF)
    w = _w(m=2, n=1, k=64, lda=2, ldb=64, op_a="N", type_a="e4m3", type_b="e4m3", a=a, b=b, sfa=sfa, ld_sfa=16,
           sfb=sfb, ld_sfb=16)
    assert compare.operand_max_abs(w, "a") == 56.0
    assert compare.operand_max_abs(w, "b") == 1.0


def test_operand_max_fp6_packed():
    # B: one row of 64 E3M2 codes, bit-packed; code 0b011111 (28) at K 9 and
    # 0b000001 (0.0625) at K 40; no scales (plain fp6 takes no per-tensor
    # scale either: b_scale = 8 is ignored) -> 28
    acc = (0b011111 << (6 * 9)) | (0b000001 << (6 * 40))
    b = np.frombuffer(acc.to_bytes(48, "little"), np.uint8).reshape(1, 48).copy()
    a = np.zeros((1, 48), np.uint8)
    w = _w(k=64, lda=64, ldb=64, type_a="e3m2", type_b="e3m2", a=a, b=b, b_scale=8.0)
    assert compare.operand_max_abs(w, "b") == 28.0
    assert compare.operand_max_abs(w, "a") == 0.0
