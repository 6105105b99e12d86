"""Pins for the CPU oracle: decoders, indexing, block scales, epilogue.

None of these re-types the oracle's formulas.  They check it against what the
pages and the mathematics fix independently: the format table on the page
(bit counts), library conversions (numpy float16, torch bfloat16 / float8),
identity and permutation matrices, rank-1 closed forms, exact rational brute
force on tiny inputs, block-scale closed forms and the epilogue's special
cases.
"""
import math
import os
import zlib
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle import compare

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ------------------------------------------------------------- decoders

def _format_table():
    rows = {}
    for line in open(os.path.join(GOLDEN, "narrow_formats.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        if len(parts) == 5:
            rows[parts[0]] = dict(e=int(parts[1]), m=int(parts[2]), signed=parts[3] == "yes",
                                  bits=int(parts[4]))
    return rows


def _minifloat(code, e_bits, m_bits, signed):
    """Generic sign/exponent/mantissa value with bias 2^(e-1)-1 and gradual
    underflow; special encodings are the caller's business."""
    bias = 2 ** (e_bits - 1) - 1
    s = (code >> (e_bits + m_bits)) & 1 if signed else 0
    e = (code >> m_bits) & ((1 << e_bits) - 1)
    f = code & ((1 << m_bits) - 1)
    if e == 0:
        mag = Fraction(f, 2 ** m_bits) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(f, 2 ** m_bits)) * Fraction(2) ** (e - bias)
    return -mag if s else mag


def test_format_table_fixture_has_the_hot_path_types():
    t = _format_table()
    assert t["float_e4m3_t"] == dict(e=4, m=3, signed=True, bits=8)
    assert t["float_e2m1_t"] == dict(e=2, m=1, signed=True, bits=4)
    assert t["float_ue8m0_t"] == dict(e=8, m=0, signed=False, bits=8)


def test_e4m3_matches_table_bit_counts():
    spec = _format_table()["float_e4m3_t"]
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e4m3", codes)
    for c in range(256):
        if (c & 0x7F) == 0x7F:  # OCP E4M3: S.1111.111 is the only NaN, no infinities
            assert math.isnan(got[c])
        else:
            assert Fraction(got[c]) == _minifloat(c, spec["e"], spec["m"], spec["signed"]), hex(c)


def test_e5m2_matches_table_bit_counts():
    spec = _format_table()["float_e5m2_t"]
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e5m2", codes)
    for c in range(256):
        if (c & 0x7C) == 0x7C:  # OCP E5M2 keeps the IEEE specials: exponent 31 is inf (mantissa 0) or NaN
            if c & 3:
                assert math.isnan(got[c])
            else:
                assert got[c] == (-math.inf if c & 0x80 else math.inf)
        else:
            assert Fraction(got[c]) == _minifloat(c, spec["e"], spec["m"], spec["signed"]), hex(c)


def test_e2m1_matches_table_bit_counts():
    spec = _format_table()["float_e2m1_t"]
    codes = np.arange(256, dtype=np.uint8)  # each byte holds two codes
    got = oracle.decode("e2m1", codes)
    for byte in range(256):
        lo, hi = byte & 0xF, byte >> 4
        assert Fraction(got[2 * byte]) == _minifloat(lo, spec["e"], spec["m"], spec["signed"])
        assert Fraction(got[2 * byte + 1]) == _minifloat(hi, spec["e"], spec["m"], spec["signed"])


def test_e2m1_magnitudes():
    got = oracle.decode("e2m1", np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], np.uint8))
    assert list(got[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(got[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


def test_e8m0_is_a_power_of_two_with_bias_127():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e8m0", codes)
    lib = codes.view(np.uint8)
    ref = torch.from_numpy(lib.copy()).view(torch.float8_e8m0fnu).double().numpy()
    for c in range(255):
        assert got[c] == 2.0 ** (c - 127)
        assert got[c] == ref[c]
    assert math.isnan(got[255]) and math.isnan(ref[255])


def test_f16_all_codes_match_numpy():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("f16", codes)
    ref = codes.view(np.float16).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("bf16", codes)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e4m3", codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e5m2_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode("e5m2", codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).double().numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e5m2_hand_points():
    got = oracle.decode("e5m2", np.array([0x3C, 0xBC, 0x7B, 0x04, 0x01, 0x7C, 0xFC, 0x7D, 0x00], np.uint8))
    assert list(got[:7]) == [1.0, -1.0, 57344.0, 2.0 ** -14, 2.0 ** -16, math.inf, -math.inf]
    assert math.isnan(got[7]) and got[8] == 0.0


def test_e4m3_hand_points():
    got = oracle.decode("e4m3", np.array([0x38, 0xB8, 0x7E, 0x08, 0x01, 0x7F, 0xFF, 0x00], np.uint8))
    assert list(got[:5]) == [1.0, -1.0, 448.0, 2.0 ** -6, 2.0 ** -9]
    assert math.isnan(got[5]) and math.isnan(got[6]) and got[7] == 0.0


def test_f32_spot_values():
    vals = np.array([1.0, -2.5, 3.0e-45, 1.0e38, 0.0], dtype=np.float32)
    assert list(oracle.decode("f32", vals.view(np.uint32))) == [float(v) for v in vals]


# ------------------------------------------------------------- GEMM helpers

def _problem(fmt, a_log, b_log, op_a="T", op_b="N", pad=0, **kw):
    """Store logical op(A) (M x K) and op(B) (K x N) in format fmt."""
    m, k = a_log.shape
    n = b_log.shape[1]
    sa = a_log if op_a == "N" else a_log.T
    sb = b_log if op_b == "N" else b_log.T
    lda = max(1, sa.shape[0]) + pad
    ldb = max(1, sb.shape[0]) + pad
    if fmt == "e2m1":
        assert op_a == "T" and op_b == "N"
        lda += lda % 2
        ldb += ldb % 2
        a = wl.pack_e2m1(wl.store_colmajor(wl.encode_e2m1_codes(sa), lda))
        b = wl.pack_e2m1(wl.store_colmajor(wl.encode_e2m1_codes(sb), ldb))
    else:
        a = wl.store_colmajor(wl.encode(sa, fmt), lda)
        b = wl.store_colmajor(wl.encode(sb, fmt), ldb)
    p = dict(m=m, n=n, k=k, a=a, lda=lda, op_a=op_a, type_a=fmt, b=b, ldb=ldb, op_b=op_b,
             type_b=fmt)
    p.update(kw)
    return p


def _values(fmt, x):
    """Round to fmt through the generator's encoder and back via a library."""
    if fmt == "f16":
        return x.astype(np.float16).astype(np.float64)
    if fmt == "bf16":
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    if fmt == "e4m3":
        return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    if fmt == "e5m2":
        return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e5m2).double().numpy()
    if fmt == "i8":
        return x.astype(np.int8).astype(np.float64)
    if fmt == "e2m1":
        return x  # tests pass exact E2M1 values
    raise ValueError(fmt)


def _random_values(fmt, g, shape):
    if fmt == "i8":
        return g.integers(-128, 128, size=shape).astype(np.float64)
    if fmt == "e2m1":
        return g.choice(np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6]),
                        size=shape)
    if fmt == "e4m3":
        return _values(fmt, g.standard_normal(shape) * 20)
    if fmt == "e5m2":
        return _values(fmt, g.standard_normal(shape) * 1000)
    return _values(fmt, g.uniform(-1, 1, size=shape))


FLOAT_FMTS = ["f16", "bf16", "e4m3", "e5m2", "e2m1"]
ALL_FMTS = FLOAT_FMTS + ["i8"]


def _full(p):
    return oracle.gemm_full(p)


def _unit_scales(rows, k):
    kb = max(1, k // 32)
    return np.full((rows, kb), 127, np.uint8), kb


# ------------------------------------------------------------- GEMM pins

@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_identity_a_returns_b(fmt):
    g = np.random.default_rng(1)
    k = 64
    n = 40
    b = _random_values(fmt, g, (k, n))
    kw = {}
    if fmt == "e2m1":
        kw["sfa"], kw["ld_sfa"] = _unit_scales(k, k)
        kw["sfb"], kw["ld_sfb"] = _unit_scales(n, k)
    p = _problem(fmt, np.eye(k), b, **kw)
    d = _full(p)
    assert np.array_equal(d, b.astype(d.dtype))


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_permutation_a_permutes_rows_of_b(fmt):
    g = np.random.default_rng(2)
    k, n = 64, 24
    perm = g.permutation(k)
    a = np.zeros((k, k))
    a[np.arange(k), perm] = 1.0
    b = _random_values(fmt, g, (k, n))
    kw = {}
    if fmt == "e2m1":
        kw["sfa"], kw["ld_sfa"] = _unit_scales(k, k)
        kw["sfb"], kw["ld_sfb"] = _unit_scales(n, k)
    d = _full(_problem(fmt, a, b, **kw))
    assert np.array_equal(d, b[perm].astype(d.dtype))


@pytest.mark.parametrize("fmt", ["f16", "bf16", "e4m3", "e5m2", "i8"])
@pytest.mark.parametrize("ops", [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")])
def test_storage_op_does_not_change_the_result(fmt, ops):
    g = np.random.default_rng(3)
    m, n, k = 7, 5, 9
    a, b = _random_values(fmt, g, (m, k)), _random_values(fmt, g, (k, n))
    ref = _full(_problem(fmt, a, b, "T", "N"))
    got = _full(_problem(fmt, a, b, ops[0], ops[1], pad=3))
    assert np.array_equal(ref, got)


def test_rank_one_closed_form_with_epilogue():
    # A(i,p) = u_i, B(p,j) = v_j with dyadic u, v: D = alpha*K*u_i*v_j + beta*C + bias
    m, n, k = 6, 5, 96
    u = np.array([0.5, -0.25, 1.0, 0.75, -1.0, 0.125])
    v = np.array([0.5, 1.0, -0.5, 0.25, -0.75])
    a = np.repeat(u[:, None], k, axis=1)
    b = np.repeat(v[None, :], k, axis=0)
    c = np.arange(m * n, dtype=np.float64).reshape(m, n) / 8 - 1
    bias = np.linspace(-1, 1, m)
    p = _problem("bf16", a, b, "N", "N", alpha=2.0, beta=-0.5,
                 c=wl.store_colmajor(c.astype(np.float32).view(np.uint32), m), ldc=m,
                 type_c="f32", bias=bias.astype(np.float32).view(np.uint32), type_bias="f32")
    want = 2.0 * k * np.outer(u, v) - 0.5 * c + bias.astype(np.float32)[:, None]
    assert np.array_equal(_full(p), want)


def test_fp8_per_tensor_scales_multiply_the_sum():
    m, n, k = 4, 3, 128
    a = np.ones((m, k))
    b = np.ones((k, n)) * 2
    p = _problem("e4m3", a, b, a_scale=0.375, b_scale=1.5, alpha=2.0)
    assert np.array_equal(_full(p), np.full((m, n), 2.0 * 0.375 * 1.5 * 2 * k))


def _exact_reference(fmt, a_vals, b_vals, *, alpha=1, beta=0, c=None, bias=None, act="none",
                     sfa=None, sfb=None):
    """Exact rational evaluation with numpy object matrices (library matmul of
    Fractions), independent of the oracle's indexing."""
    fa = np.vectorize(Fraction, otypes=[object])(a_vals)
    fb = np.vectorize(Fraction, otypes=[object])(b_vals)
    if sfa is not None:
        k = a_vals.shape[1]
        blk = np.arange(k) // 32
        fa = fa * np.vectorize(lambda e: Fraction(2) ** (int(e) - 127), otypes=[object])(sfa[:, blk])
        fb = fb * np.vectorize(lambda e: Fraction(2) ** (int(e) - 127), otypes=[object])(sfb[:, blk]).T
    acc = fa.dot(fb)
    t = acc * Fraction(alpha)
    if beta:
        t = t + Fraction(beta) * np.vectorize(Fraction, otypes=[object])(c)
    if bias is not None:
        t = t + np.vectorize(Fraction, otypes=[object])(bias)[:, None]
    if act == "relu":
        t = np.vectorize(lambda x: max(x, Fraction(0)), otypes=[object])(t)
    return t


@pytest.mark.parametrize("fmt", FLOAT_FMTS)
@pytest.mark.parametrize("trial", range(4))
def test_bruteforce_exact_on_tiny_inputs(fmt, trial):
    g = np.random.default_rng(100 + trial)
    m, n = int(g.integers(1, 7)), int(g.integers(1, 7))
    k = 64 if fmt == "e2m1" else int(g.integers(1, 7))
    a, b = _random_values(fmt, g, (m, k)), _random_values(fmt, g, (k, n))
    kw, ex = {}, {}
    if fmt == "e2m1":
        sfa = g.integers(120, 135, size=(m, k // 32)).astype(np.uint8)
        sfb = g.integers(120, 135, size=(n, k // 32)).astype(np.uint8)
        kw = dict(sfa=sfa, ld_sfa=k // 32, sfb=sfb, ld_sfb=k // 32)
        ex = dict(sfa=sfa, sfb=sfb)
    c = _values("bf16", g.uniform(-4, 4, size=(m, n)))
    bias = _values("bf16", g.uniform(-2, 2, size=m))
    act = ["none", "relu"][trial % 2]
    p = _problem(fmt, a, b, "T", "N", alpha=1.5, beta=-0.75,
                 c=wl.store_colmajor(wl.encode(c, "bf16"), m), ldc=m, type_c="bf16",
                 bias=wl.encode(bias, "bf16"), type_bias="bf16", act=act, **kw)
    got = _full(p)
    want = _exact_reference(fmt, a, b, alpha=1.5, beta=-0.75, c=c, bias=bias, act=act, **ex)
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(got[i, j]) - want[i, j]) <= Fraction(2) ** -48 * (1 + abs(want[i, j]))


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("trial", range(3))
def test_bruteforce_exact_mxfp8(trial, fa, fb):
    # fp8 elements (E4M3, E5M2, or one of each) with E8M0 block scales (MX
    # fp8): the block-scaled sum is the same definition as for e2m1, now over
    # 8-bit elements, each operand decoded by its own format
    g = np.random.default_rng(300 + trial)
    m, n, k = int(g.integers(1, 6)), int(g.integers(1, 6)), 96
    a, b = _random_values(fa, g, (m, k)), _random_values(fb, g, (k, n))
    sfa = g.integers(118, 136, size=(m, k // 32)).astype(np.uint8)
    sfb = g.integers(118, 136, size=(n, k // 32)).astype(np.uint8)
    p = dict(m=m, n=n, k=k, a=wl.store_colmajor(wl.encode(a.T, fa), k), lda=k, op_a="T", type_a=fa,
             b=wl.store_colmajor(wl.encode(b, fb), k), ldb=k, op_b="N", type_b=fb, alpha=0.75, a_scale=2.0,
             b_scale=0.5, sfa=sfa, ld_sfa=k // 32, sfb=sfb, ld_sfb=k // 32)
    got = _full(p)
    want = _exact_reference(fa, a, b, alpha=0.75, sfa=sfa, sfb=sfb)  # a_scale * b_scale = 1
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(got[i, j]) - want[i, j]) <= Fraction(2) ** -48 * (1 + abs(want[i, j]))


@pytest.mark.parametrize("fa,fb", [("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_mixed_fp8_bruteforce_exact(fa, fb):
    # A and B in different fp8 formats: each operand decoded by its own format
    g = np.random.default_rng(500)
    m, n, k = 4, 5, 7
    a, b = _random_values(fa, g, (m, k)), _random_values(fb, g, (k, n))
    p = dict(m=m, n=n, k=k, a=wl.store_colmajor(wl.encode(a.T, fa), k), lda=k, op_a="T", type_a=fa,
             b=wl.store_colmajor(wl.encode(b, fb), k), ldb=k, op_b="N", type_b=fb, alpha=1.25, a_scale=0.5,
             b_scale=4.0)
    got = _full(p)
    want = _exact_reference(fa, a, b, alpha=2.5)  # 1.25 * 0.5 * 4
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(got[i, j]) - want[i, j]) <= Fraction(2) ** -48 * (1 + abs(want[i, j]))


def test_bruteforce_int8_exact():
    g = np.random.default_rng(7)
    for _ in range(5):
        m, n, k = (int(x) for x in g.integers(1, 9, size=3))
        a, b = _random_values("i8", g, (m, k)), _random_values("i8", g, (k, n))
        c = g.integers(-5000, 5000, size=(m, n)).astype(np.int32)
        bias = g.integers(-5000, 5000, size=m).astype(np.int32)
        p = _problem("i8", a, b, "T", "N", beta=1.0, c=wl.store_colmajor(c, m), ldc=m,
                     type_c="i32", bias=bias, type_bias="i32")
        want = a.astype(np.int64) @ b.astype(np.int64) + c + bias[:, None]
        assert np.array_equal(_full(p), want)


def test_bruteforce_int8_relu_exact():
    # The integer epilogue with relu: sums of both signs, C and bias, against
    # exact int64 arithmetic and max(t, 0).  C and bias are drawn so that
    # about half of the outputs are negative before the activation.
    g = np.random.default_rng(11)
    for _ in range(5):
        m, n, k = (int(x) for x in g.integers(2, 9, size=3))
        a, b = _random_values("i8", g, (m, k)), _random_values("i8", g, (k, n))
        c = g.integers(-30000, 30000, size=(m, n)).astype(np.int32)
        bias = g.integers(-30000, 30000, size=m).astype(np.int32)
        p = _problem("i8", a, b, "T", "N", beta=1.0, c=wl.store_colmajor(c, m), ldc=m,
                     type_c="i32", bias=bias, type_bias="i32", act="relu")
        t = a.astype(np.int64) @ b.astype(np.int64) + c + bias[:, None]
        assert (t < 0).any() and (t > 0).any()
        assert np.array_equal(_full(p), np.maximum(t, 0))


def test_int8_relu_boundary_points():
    # t = -1, 0, +1 exactly (A = 0): relu gives 0, 0, 1
    m, n, k = 3, 1, 4
    c = np.array([[-1], [0], [1]], np.int32)
    p = _problem("i8", np.zeros((m, k)), np.zeros((k, n)), beta=1.0,
                 c=wl.store_colmajor(c, m), ldc=m, type_c="i32", act="relu")
    assert np.array_equal(_full(p)[:, 0], np.array([0, 0, 1]))


def test_block_scale_closed_form():
    # A = B = all 1.0 (code 0x2), SFA(i,kb) = 2^((i+kb) mod 3), SFB(j,kb) = 2^(j mod 2):
    # D(i,j) = 32 * 2^(j mod 2) * sum_kb 2^((i+kb) mod 3).  A block boundary off by
    # one, a swapped row/column or a swapped operand changes the value.
    m, n, k = 5, 4, 256
    kb = k // 32
    sfa = np.array([[127 + (i + q) % 3 for q in range(kb)] for i in range(m)], np.uint8)
    sfb = np.array([[127 + j % 2 for _ in range(kb)] for j in range(n)], np.uint8)
    p = _problem("e2m1", np.ones((m, k)), np.ones((k, n)), sfa=sfa, ld_sfa=kb, sfb=sfb,
                 ld_sfb=kb)
    want = np.array([[32 * 2 ** (j % 2) * sum(2 ** ((i + q) % 3) for q in range(kb))
                      for j in range(n)] for i in range(m)], dtype=np.float64)
    assert np.array_equal(_full(p), want)


def test_block_scale_changes_only_its_own_block():
    m, n, k = 1, 1, 128
    sfa = np.full((m, 4), 127, np.uint8)
    sfa[0, 2] = 130  # block 2 (k = 64..95) scaled by 8
    sfb = np.full((n, 4), 127, np.uint8)
    a = np.zeros((m, k))
    a[0, 63], a[0, 64], a[0, 95], a[0, 96] = 1.0, 1.0, 1.0, 1.0
    p = _problem("e2m1", a, np.ones((k, n)), sfa=sfa, ld_sfa=4, sfb=sfb, ld_sfb=4)
    assert _full(p)[0, 0] == 1 + 8 + 8 + 1


def test_e2m1_nibble_order():
    # A one-hot at k=0 lives in the low nibble of byte 0, k=1 in its high nibble.
    m, n, k = 1, 1, 32
    b = np.zeros((k, n))
    b[0, 0], b[1, 0] = 2.0, 3.0
    for hot, want in ((0, 2.0), (1, 3.0)):
        a = np.zeros((m, k))
        a[0, hot] = 1.0
        p = _problem("e2m1", a, b, sfa=np.full((1, 1), 127, np.uint8), ld_sfa=1,
                     sfb=np.full((1, 1), 127, np.uint8), ld_sfb=1)
        assert p["a"][0, 0] == (0x02 if hot == 0 else 0x20)
        assert _full(p)[0, 0] == want


@pytest.mark.parametrize("act", ["none", "relu", "gelu"])
def test_zero_a_gives_activation_of_c_plus_bias(act):
    m, n, k = 8, 3, 16
    t = np.linspace(-6, 6, m * n).reshape(m, n)
    bias = np.linspace(-0.5, 0.5, m)
    p = _problem("bf16", np.zeros((m, k)), np.ones((k, n)), beta=2.0,
                 c=wl.store_colmajor(t.astype(np.float32).view(np.uint32), m), ldc=m,
                 type_c="f32", bias=bias.astype(np.float32).view(np.uint32), type_bias="f32",
                 act=act)
    x = 2.0 * t.astype(np.float32).astype(np.float64) + bias.astype(np.float32)[:, None]
    got = _full(p)
    if act == "none":
        assert np.array_equal(got, x)
    elif act == "relu":
        assert np.array_equal(got, np.maximum(x, 0))
    else:
        ref = np.vectorize(lambda v: 0.5 * v * (1 + math.erf(v / math.sqrt(2))))(x)
        assert np.allclose(got, ref, rtol=1e-15, atol=1e-300)


def test_gelu_special_points():
    m, n, k = 3, 1, 1
    c = np.array([[0.0], [20.0], [-20.0]])
    p = _problem("bf16", np.zeros((m, k)), np.zeros((k, n)), beta=1.0,
                 c=wl.store_colmajor(c.astype(np.float32).view(np.uint32), m), ldc=m,
                 type_c="f32", act="gelu")
    got = _full(p)[:, 0]
    assert got[0] == 0.0 and got[1] == 20.0 and abs(got[2]) < 1e-80


def _normal_cdf_table():
    rows = []
    for line in open(os.path.join(GOLDEN, "normal_cdf.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            x, phi = line.split()
            rows.append((float(x), float(phi)))
    return rows


def test_normal_cdf_table_matches_an_independent_implementation():
    from scipy.special import ndtr

    for x, phi in _normal_cdf_table():
        assert abs(float(ndtr(x)) - phi) <= 1e-15


def test_gelu_is_x_times_the_normal_cdf():
    # GELU (erf form) at mid-range points: D = x * Phi(x) with Phi from the
    # tabulated standard normal distribution, to 1e-14 absolute.  The tanh
    # approximation misses these by 2e-5 or more; a wrong argument scale
    # (erf(x/2)) or a missing factor 1/2 by far more.
    tab = _normal_cdf_table()
    m, n, k = len(tab), 1, 1
    c = np.array([[x] for x, _ in tab])
    p = _problem("bf16", np.zeros((m, k)), np.zeros((k, n)), beta=1.0,
                 c=wl.store_colmajor(c.astype(np.float32).view(np.uint32), m), ldc=m,
                 type_c="f32", act="gelu")
    got = _full(p)[:, 0]
    for (x, phi), d in zip(tab, got):
        assert abs(d - x * phi) <= 1e-14, (x, d, x * phi)


def test_gelu_matches_torch_exact_gelu():
    # torch's own erf-form GELU (approximate='none') in float64 on the CPU, an
    # implementation independent of the oracle's, at 64 points over [-6, 6].
    x = np.linspace(-6.0, 6.0, 64).astype(np.float32).astype(np.float64)
    m, n, k = x.size, 1, 1
    p = _problem("bf16", np.zeros((m, k)), np.zeros((k, n)), beta=1.0,
                 c=wl.store_colmajor(x[:, None].astype(np.float32).view(np.uint32), m), ldc=m,
                 type_c="f32", act="gelu")
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.allclose(_full(p)[:, 0], ref, rtol=1e-14, atol=1e-300)


def test_relu_boundary_points():
    m, n, k = 3, 1, 1
    c = np.array([[-1.0], [0.0], [1.0]])
    p = _problem("bf16", np.zeros((m, k)), np.zeros((k, n)), beta=1.0,
                 c=wl.store_colmajor(c.astype(np.float32).view(np.uint32), m), ldc=m,
                 type_c="f32", act="relu")
    assert list(_full(p)[:, 0]) == [0.0, 0.0, 1.0]


def test_beta_zero_ignores_c():
    m, n, k = 2, 2, 4
    nan_c = np.full((n, m), np.float32(np.nan)).view(np.uint32)
    p = _problem("f16", np.ones((m, k)), np.ones((k, n)), beta=0.0, c=nan_c, ldc=m, type_c="f32")
    assert np.array_equal(_full(p), np.full((m, n), 4.0))


@pytest.mark.parametrize("va,vb", [(127, 127), (-128, -128), (127, -128)])
def test_int8_extremes(va, vb):
    m, n, k = 3, 4, 4096
    p = _problem("i8", np.full((m, k), va), np.full((k, n), vb))
    assert np.array_equal(_full(p), np.full((m, n), k * va * vb, dtype=np.int64))


def test_k_zero_gives_epilogue_only():
    m, n = 3, 2
    c = np.arange(6, dtype=np.float32).reshape(m, n)
    p = _problem("f16", np.zeros((m, 0)), np.zeros((0, n)), beta=1.0,
                 c=wl.store_colmajor(c.view(np.uint32), m), ldc=m, type_c="f32", act="relu")
    assert np.array_equal(_full(p), c.astype(np.float64))


def test_oracle_rejects_out_of_range_requests():
    p = _problem("f16", np.ones((2, 2)), np.ones((2, 2)))
    with pytest.raises(ValueError):
        oracle.gemm_elements(p, [2], [0])


def test_threads_do_not_change_results():
    w = wl.make("bf16", 40, 30, 50)
    p = w.oracle_problem()
    assert np.array_equal(oracle.gemm_full(p, nthreads=1), oracle.gemm_full(p, nthreads=4))


# ------------------------------------------------------------- tolerance

def test_ulp_out_values():
    assert compare.ulp_out("bf16", 1.0) == 2.0 ** -7
    assert compare.ulp_out("bf16", 1.99) == 2.0 ** -7
    assert compare.ulp_out("bf16", 2.0) == 2.0 ** -6
    assert compare.ulp_out("f32", 1.0) == 2.0 ** -23
    assert compare.ulp_out("f32", 0.0) == 2.0 ** -149
    assert compare.ulp_out("f16", 1e-7) == 2.0 ** -24
    assert compare.ulp_out("f16", 1024.0) == 1.0


def test_fp32_accumulation_stays_well_inside_the_bound():
    # Diagnostic for the tolerance: a plain fp32 CPU dot product over K = 4096
    # of U[-1,1] bf16 operands is far inside 2^-20 * K * max|a| * max|b|.
    w = wl.make("bf16", 32, 32, 4096, beta=0.0, bias=False, act="none")
    a = oracle.decode("bf16", w.a).reshape(w.k, w.lda)[:, : w.m].T  # op N: stored M x K
    b = oracle.decode("bf16", w.b).reshape(w.n, w.ldb)[:, : w.k].T
    ref = oracle.gemm_full(w.oracle_problem())
    f32 = (a.astype(np.float32) @ b.astype(np.float32)).astype(np.float64)
    bound = 2.0 ** -20 * w.k * np.abs(a).max() * np.abs(b).max()
    assert np.abs(f32 - ref).max() < bound / 8


# ------------------------------------------------------------- MX output blocks

def test_mx_all_equal_block():
    # 32 x 1.0: amax 1, X = 0 - emax; every element is 2^emax in the format
    for fmt, emax, code in (("e2m1", 2, 0x6), ("e4m3", 8, 0x78), ("e5m2", 15, 0x78)):
        codes, sc = oracle.mx_quantize_block([1.0] * 32, fmt)
        assert sc == 127 - emax and (codes == code).all(), (fmt, sc, codes)


def test_mx_e2m1_ties_go_to_the_even_code_and_large_values_saturate():
    # amax 7 -> X = floor(log2 7) - 2 = 0: values are quantized as they are.
    vals = [7.0, 5.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -3.5, 6.0, -0.5, 0.1]
    codes, sc = oracle.mx_quantize_block(vals, "e2m1")
    assert sc == 127
    # 7 -> 6 (clamped); 5 -> 4; 0.25 -> 0; 0.75 -> 1; 1.25 -> 1; 1.75 -> 2; 2.5 -> 2;
    # 3.5 -> 4; -3.5 -> -4; 6 -> 6; -0.5 -> -0.5; 0.1 -> 0
    assert codes.tolist() == [0x7, 0x6, 0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0xE, 0x7, 0x9, 0x0]


def test_mx_scale_follows_the_binade_of_amax():
    # just below a power of two stays in the lower binade; the power itself moves up
    _, s1 = oracle.mx_quantize_block([8.0 - 2.0 ** -20, 1.0], "e2m1")
    _, s2 = oracle.mx_quantize_block([8.0, 1.0], "e2m1")
    _, s3 = oracle.mx_quantize_block([-8.0, 1.0], "e2m1")
    assert (s1, s2, s3) == (127, 128, 128)
    # the scale code saturates at both ends of E8M0
    c_hi, s_hi = oracle.mx_quantize_block([2.0 ** 200, -(2.0 ** 199)], "e2m1")
    c_lo, s_lo = oracle.mx_quantize_block([2.0 ** -200, -(2.0 ** -201)], "e2m1")
    assert s_hi == 254 and c_hi.tolist() == [0x7, 0xF]  # 2^73 and -2^72 clamp to +-6
    assert s_lo == 0 and c_lo.tolist() == [0x0, 0x8]    # far below the smallest element: signed zeros


def test_mx_zero_block():
    codes, sc = oracle.mx_quantize_block([0.0, -0.0, 0.0], "e4m3")
    assert sc == 0 and codes.tolist() == [0x00, 0x80, 0x00]


def test_mx_e4m3_subnormal_elements():
    # amax 1 -> X = -8; 2^-17 / 2^-8 = 2^-9 is E4M3's smallest subnormal (code 1);
    # 1.5 * 2^-9 is a tie between codes 1 and 2 -> 2; 448.5 * 2^-8 clamps to 448 (0x7E)
    codes, sc = oracle.mx_quantize_block([1.0, 2.0 ** -17, 1.5 * 2.0 ** -17, 2.0 ** -30], "e4m3")
    assert sc == 119 and codes.tolist() == [0x78, 0x01, 0x02, 0x00]
    codes, sc = oracle.mx_quantize_block([511.0 * 2.0 ** -8, 1.0], "e4m3")
    assert sc == 119 and codes.tolist() == [0x7E, 0x78]


def test_mx_e5m2_saturates_below_its_infinity():
    # amax 65535 -> X = 15 - 15 = 0: 65535 clamps to 57344 (0x7B), never to the Inf code 0x7C
    codes, sc = oracle.mx_quantize_block([65535.0, -40000.0, 1.0], "e5m2")
    assert sc == 127 and codes.tolist() == [0x7B, 0xF9, 0x3C]


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3", "e5m2"])
def test_mx_blocks_dequantize_within_half_a_step(fmt):
    # every element dequantizes to within half the element grid's spacing at
    # its magnitude (times 2^X), except values above the largest element,
    # which clamp to it; and the scale puts amax in the top binade
    top = {"e2m1": 6.0, "e4m3": 448.0, "e5m2": 57344.0}[fmt]
    emax = {"e2m1": 2, "e4m3": 8, "e5m2": 15}[fmt]
    dec = {"e2m1": lambda c: oracle.decode("e2m1", np.array([c | (c << 4)], np.uint8))[0],
           "e4m3": lambda c: oracle.decode("e4m3", np.array([c], np.uint8))[0],
           "e5m2": lambda c: oracle.decode("e5m2", np.array([c], np.uint8))[0]}[fmt]
    mags = [abs(dec(c)) for c in range(8 if fmt == "e2m1" else 256)]
    grid = np.array(sorted({v for v in mags if np.isfinite(v)}))
    g = np.random.default_rng(17)
    for trial in range(50):
        vals = g.standard_normal(32) * np.exp(g.uniform(-30, 30))
        codes, sc = oracle.mx_quantize_block(vals, fmt)
        x = sc - 127
        amax = np.abs(vals).max()
        assert 2.0 ** (x + emax) <= amax < 2.0 ** (x + emax + 1)
        for v, c in zip(vals, codes):
            a = abs(v) / 2.0 ** x
            got = abs(dec(int(c) & (0x7 if fmt == "e2m1" else 0x7F)))
            assert (c >> (3 if fmt == "e2m1" else 7)) == (v < 0)
            if a >= top:
                assert got == top
            else:
                i = np.searchsorted(grid, a)
                lo, hi = grid[max(i - 1, 0)], grid[min(i, grid.size - 1)]
                assert got in (lo, hi) and abs(got - a) <= (hi - lo) / 2 + 1e-300


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3", "e5m2"])
def test_mx_blocks_agree_with_the_input_generators_quantizer(fmt):
    # the generators' numpy quantizer (an independent implementation of the
    # same OCP rule, used to make the MX operands) gives the same scales and
    # elements on random blocks
    g = np.random.default_rng(18)
    x = g.standard_normal((8, 64)) * np.exp(g.uniform(-10, 10, size=(8, 1)))
    if fmt == "e2m1":
        want_codes, want_sc = wl.mx_quantize(x)
    else:
        want_codes, want_sc = wl.mx_quantize_fp8(x, fmt)
    for r in range(8):
        for b in range(2):
            codes, sc = oracle.mx_quantize_block(x[r, 32 * b: 32 * b + 32], fmt)
            assert sc == want_sc[r, b]
            assert codes.tolist() == want_codes[r, 32 * b: 32 * b + 32].tolist()


# ------------------------------------------------------------- fp6 and mixed narrow formats

def _fp6_stream(codes):
    """Bytes of 6-bit codes laid out as one little-endian bit stream (element
    t in bits 6t .. 6t+5), built with Python integers."""
    acc = 0
    for t, c in enumerate(codes):
        acc |= int(c) << (6 * t)
    nbytes = (6 * len(codes) + 7) // 8
    return np.frombuffer(acc.to_bytes(nbytes, "little"), dtype=np.uint8).copy()


@pytest.mark.parametrize("fmt,table", [("e2m3", "float_e2m3_t"), ("e3m2", "float_e3m2_t")])
def test_fp6_matches_table_bit_counts(fmt, table):
    # every one of the 64 codes: the table's exponent and mantissa widths,
    # bias 2^(e-1) - 1, gradual underflow, no special encodings (OCP fp6)
    spec = _format_table()[table]
    assert spec["bits"] == 6 and spec["signed"]
    got = oracle.decode(fmt, _fp6_stream(range(64)), 64)
    for c in range(64):
        assert Fraction(got[c]) == _minifloat(c, spec["e"], spec["m"], True), (fmt, c)


@pytest.mark.parametrize("fmt,extremes", [
    # OCP MX specification, fp6 format table: max normal, min normal, max subnormal, min subnormal
    ("e2m3", (7.5, 1.0, 0.875, 0.125)),
    ("e3m2", (28.0, 0.25, 0.1875, 0.0625)),
])
def test_fp6_published_extremes(fmt, extremes):
    e_bits = 2 if fmt == "e2m3" else 3
    m_bits = 5 - e_bits
    max_norm = 0b011111
    min_norm = 1 << m_bits
    max_sub = (1 << m_bits) - 1
    got = oracle.decode(fmt, _fp6_stream([max_norm, min_norm, max_sub, 1]), 4)
    assert tuple(got) == extremes
    neg = oracle.decode(fmt, _fp6_stream([32 | max_norm]), 1)
    assert neg[0] == -extremes[0]


def test_fp6_packing_by_hand():
    # E2M3 codes 0b000001 (0.125), 0b011111 (7.5), 0b100000 (-0), 0b111111 (-7.5)
    # in one 24-bit little-endian word: 0xFE07C1 -> bytes C1 07 FE
    got = oracle.decode("e2m3", np.array([0xC1, 0x07, 0xFE], np.uint8), 4)
    assert list(got) == [0.125, 7.5, 0.0, -7.5] and math.copysign(1, got[2]) == -1
    # an element straddling a byte: element 1 of E3M2 occupies bits 6 .. 11
    got = oracle.decode("e3m2", np.array([0b11000000, 0b00000111, 0], np.uint8), 4)
    assert list(got) == [0.0, 28.0, 0.0, 0.0]


def _narrow_values(fmt, g, shape):
    """Random exact values of a narrow format and their stored codes, from
    the format table's bit counts (codes first, values by _minifloat)."""
    spec = {"e4m3": (4, 3, 8), "e5m2": (5, 2, 8), "e2m3": (2, 3, 6), "e3m2": (3, 2, 6), "e2m1": (2, 1, 4)}[fmt]
    e_bits, m_bits, bits = spec
    codes = g.integers(0, 1 << bits, size=shape)
    if fmt == "e4m3":  # skip the NaN codes
        codes = np.where((codes & 0x7F) == 0x7F, codes ^ 1, codes)
    if fmt == "e5m2":  # and the infinities / NaNs
        codes = np.where((codes & 0x7C) == 0x7C, codes & 0x83, codes)
    vals = np.vectorize(lambda c: _minifloat(int(c), e_bits, m_bits, True), otypes=[object])(codes)
    return codes.astype(np.uint8), vals


def _stored(codes_rows, fmt, kmajor, ld):
    lines = codes_rows if kmajor else codes_rows.T
    mem = np.zeros((lines.shape[0], ld), np.uint8)
    mem[:, : lines.shape[1]] = lines
    if fmt == "e2m1":
        return wl.pack_e2m1(mem)
    if fmt in ("e2m3", "e3m2"):
        return np.concatenate([_fp6_stream(row) for row in mem]).reshape(mem.shape[0], -1)
    return mem


@pytest.mark.parametrize("fa,fb", [("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m3", "e3m2"), ("e4m3", "e2m1"),
                                   ("e2m1", "e5m2"), ("e3m2", "e4m3"), ("e2m1", "e2m3")])
@pytest.mark.parametrize("ops", [("T", "N"), ("N", "N"), ("T", "T"), ("N", "T")])
@pytest.mark.parametrize("mx", [False, True])
def test_bruteforce_exact_narrow_pairs_in_every_layout(fa, fb, ops, mx):
    # random codes of each format, stored in the given layout (fp6 packed into
    # a bit stream, fp4 two a byte), against exact rational arithmetic on the
    # values the format table defines; block scales (MX) per 32 K-elements of
    # each logical row whatever the storage
    g = np.random.default_rng(zlib.crc32(f"{fa}{fb}{ops}{mx}".encode()))
    m, n, k = 5, 3, 64
    ca, va = _narrow_values(fa, g, (m, k))
    cb, vb = _narrow_values(fb, g, (n, k))
    a_km, b_km = ops[0] == "T", ops[1] == "N"
    lda = 68 if a_km else 8
    ldb = 68 if b_km else 4
    p = dict(m=m, n=n, k=k, a=_stored(ca, fa, a_km, lda), lda=lda, op_a=ops[0], type_a=fa,
             b=_stored(cb, fb, b_km, ldb), ldb=ldb, op_b=ops[1], type_b=fb, alpha=0.5)
    ex = {}
    if mx:
        sfa = g.integers(120, 134, size=(m, k // 32)).astype(np.uint8)
        sfb = g.integers(120, 134, size=(n, k // 32)).astype(np.uint8)
        p.update(sfa=sfa, ld_sfa=k // 32, sfb=sfb, ld_sfb=k // 32)
        ex = dict(sfa=sfa, sfb=sfb)
    got = _full(p)
    want = _exact_reference(fa, va, vb.T, alpha=0.5, **ex)
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(got[i, j]) - want[i, j]) <= Fraction(2) ** -48 * (1 + abs(want[i, j])), (i, j)
