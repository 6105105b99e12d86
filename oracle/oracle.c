/*
 * oracle.c -- the plain, slow CPU oracle for the fused-epilogue GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with the
 * GPU kernels.
 *
 * What it computes, for each requested output element (i, j):
 *
 *   D(i,j) = act( alpha * s_a * s_b * sum_p a'(i,p) * b'(p,j)
 *                 + beta * C(i,j) + bias(i) )
 *
 * - The linear-combination surface alpha*op(A)*op(B) + beta*C and the BLAS
 *   column-major storage convention with op in {N, T}: "CUTLASS" knowledge-base
 *   page, opening section (the fixed cuBLAS surface) and "CuTe and layouts"
 *   (column-major strides); "Technical Documentation: NVIDIA/cutlass",
 *   "Layouts, Tensor Alignment Requirements" (T = row-major, N = column-major).
 * - The block-scaled sum a'(i,p) = A(i,p) * SFA(i, floor(p/32)), and likewise
 *   for B with SFB(j, floor(p/32)): same document, "Blackwell SM100 GEMMs",
 *   "Block Scaled GEMMs" (index-notation formula), vector size 32 for the OCP
 *   mx types ("Blackwell Block Scaled Narrow Precision Data Types" table).
 * - The element formats (e4m3, e5m2, e2m1, e2m3, e3m2, ue8m0 bit counts and
 *   signedness): same document, "Blackwell Narrow Precision Data Types" table;
 *   the bit-level meaning of each code follows the OCP formats that table
 *   points to.  The pages fix no byte packing for the 6-bit types; the reading
 *   taken is the plainest one, the same as for the 4-bit type: consecutive
 *   elements fill a little-endian bit stream, lowest bits first.
 * - The epilogue (bias, activation) applied to the GEMM result before the
 *   store: knowledge-base page, "Epilogues".
 *
 * Precision: every element is decoded to an exact double (int64 for int8);
 * the sum runs in ascending p in double (int64 for the integer path).  Every
 * product of two decoded operands is exact in double (at most 22 significant
 * bits), so the only rounding is the fp64 summation, ~1e-12 relative at
 * K = 8192.  The result is returned unrounded; rounding to the output type is
 * the comparison's business.
 *
 * Built with gcc -O2 (no fast-math) and OpenMP over output elements.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Element type codes used by this file alone. */
enum {
    ORC_F32 = 0,
    ORC_F16 = 1,
    ORC_BF16 = 2,
    ORC_I8 = 3,
    ORC_I32 = 4,
    ORC_E4M3 = 5,
    ORC_E2M1 = 6, /* two OCP fp4 codes per byte, even element in the low nibble */
    ORC_E8M0 = 7,
    ORC_E5M2 = 9,
    ORC_E2M3 = 10, /* OCP fp6 E2M3, bit-packed: element t in bits 6t .. 6t+5 of the little-endian stream */
    ORC_E3M2 = 11, /* OCP fp6 E3M2, packed the same way */
};

enum { ORC_ACT_NONE = 0, ORC_ACT_RELU = 1, ORC_ACT_GELU = 2 };

typedef struct {
    int64_t m, n, k;
    const void *a;
    int64_t lda;
    int32_t op_a; /* 0 = N: A(i,p) at a[i + p*lda];  1 = T: at a[p + i*lda] */
    int32_t type_a;
    const void *b;
    int64_t ldb;
    int32_t op_b; /* 0 = N: B(p,j) at b[p + j*ldb];  1 = T: at b[j + p*ldb] */
    int32_t type_b;
    const void *c; /* may be NULL when beta == 0 */
    int64_t ldc;   /* C(i,j) at c[i + j*ldc] */
    int32_t type_c;
    int32_t type_bias;
    const void *bias; /* length m, NULL for none */
    double alpha, beta;
    double a_scale, b_scale; /* per-tensor scales (fp8); 1 otherwise */
    const uint8_t *sfa;      /* E8M0 block scales, SFA(i,kb) at sfa[i*ld_sfa + kb]; NULL for none */
    int64_t ld_sfa;
    const uint8_t *sfb; /* SFB(j,kb) at sfb[j*ld_sfb + kb] */
    int64_t ld_sfb;
    int32_t act;
    int32_t block; /* scale-vector size along K (32 for MX) */
} oracle_problem;

/* ---------------------------------------------------------------- decoders */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double dec_f16(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24); /* subnormal: f * 2^-10 * 2^-14 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return s ? -mag : mag;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
static double dec_bf16(uint16_t h)
{
    int s = h >> 15, e = (h >> 7) & 0xff, f = h & 0x7f;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -133); /* f * 2^-7 * 2^-126 */
    else if (e == 255)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(128 + f), e - 134);
    return s ? -mag : mag;
}

/* IEEE binary32, read from its bits the same way. */
static double dec_f32(uint32_t w)
{
    int s = w >> 31, e = (w >> 23) & 0xff;
    uint32_t f = w & 0x7fffff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -149);
    else if (e == 255)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(0x800000u + f), e - 150);
    return s ? -mag : mag;
}

/* OCP E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities, S.1111.111 is NaN, largest finite magnitude 448. */
static double dec_e4m3(uint8_t q)
{
    int s = q >> 7, e = (q >> 3) & 0xf, f = q & 7;
    double mag;
    if ((q & 0x7f) == 0x7f)
        mag = NAN;
    else if (e == 0)
        mag = ldexp((double)f, -9); /* f/8 * 2^-6 */
    else
        mag = ldexp((double)(8 + f), e - 10); /* (1 + f/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* OCP E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits, with the IEEE
 * conventions: exponent 31 is infinity (mantissa 0) or NaN; largest finite
 * magnitude 1.75 * 2^15 = 57344, smallest subnormal 2^-16. */
static double dec_e5m2(uint8_t q)
{
    int s = q >> 7, e = (q >> 2) & 0x1f, f = q & 3;
    double mag;
    if (e == 31)
        mag = f == 0 ? INFINITY : NAN;
    else if (e == 0)
        mag = ldexp((double)f, -16); /* f/4 * 2^-14 */
    else
        mag = ldexp((double)(4 + f), e - 17); /* (1 + f/4) * 2^(e-15) */
    return s ? -mag : mag;
}

/* OCP E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; all codes finite. */
static double dec_e2m1(unsigned nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, f = nib & 1;
    double mag;
    if (e == 0)
        mag = 0.5 * f; /* subnormal: f/2 * 2^0 */
    else
        mag = ldexp((double)(2 + f), e - 2); /* (1 + f/2) * 2^(e-1) */
    return s ? -mag : mag;
}

/* OCP E2M3 (fp6): 1 sign, 2 exponent (bias 1), 3 mantissa bits; all codes
 * finite, largest magnitude 1.875 * 2^2 = 7.5, smallest subnormal 2^-3. */
static double dec_e2m3(unsigned c)
{
    int s = (c >> 5) & 1, e = (c >> 3) & 3, f = c & 7;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -3); /* f/8 * 2^0 */
    else
        mag = ldexp((double)(8 + f), e - 4); /* (1 + f/8) * 2^(e-1) */
    return s ? -mag : mag;
}

/* OCP E3M2 (fp6): 1 sign, 3 exponent (bias 3), 2 mantissa bits; all codes
 * finite, largest magnitude 1.75 * 2^4 = 28, smallest subnormal 2^-4. */
static double dec_e3m2(unsigned c)
{
    int s = (c >> 5) & 1, e = (c >> 2) & 7, f = c & 3;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -4); /* f/4 * 2^-2 */
    else
        mag = ldexp((double)(4 + f), e - 5); /* (1 + f/4) * 2^(e-3) */
    return s ? -mag : mag;
}

/* The 6-bit code of element idx of a bit-packed fp6 buffer: bits 6*idx ..
 * 6*idx+5 of the buffer read as one little-endian bit stream (element 0 in
 * the low six bits of byte 0; four elements fill three bytes). */
static unsigned fp6_code(const uint8_t *base, int64_t idx)
{
    int64_t bit = 6 * idx;
    int64_t byte = bit >> 3;
    int shift = (int)(bit & 7);
    unsigned w = base[byte];
    if (shift > 2)
        w |= (unsigned)base[byte + 1] << 8;
    return (w >> shift) & 63u;
}

/* OCP E8M0 scale: 8 exponent bits, bias 127, no sign or mantissa; 0xff NaN. */
static double dec_e8m0(uint8_t x)
{
    return x == 0xff ? NAN : ldexp(1.0, (int)x - 127);
}

/* Decode element `idx` (in elements) of a buffer of the given type. */
static double load_real(const void *base, int32_t type, int64_t idx)
{
    switch (type) {
    case ORC_F32: {
        uint32_t w;
        memcpy(&w, (const char *)base + 4 * idx, 4);
        return dec_f32(w);
    }
    case ORC_F16: {
        uint16_t h;
        memcpy(&h, (const char *)base + 2 * idx, 2);
        return dec_f16(h);
    }
    case ORC_BF16: {
        uint16_t h;
        memcpy(&h, (const char *)base + 2 * idx, 2);
        return dec_bf16(h);
    }
    case ORC_I8:
        return (double)((const int8_t *)base)[idx];
    case ORC_I32: {
        int32_t v;
        memcpy(&v, (const char *)base + 4 * idx, 4);
        return (double)v;
    }
    case ORC_E4M3:
        return dec_e4m3(((const uint8_t *)base)[idx]);
    case ORC_E2M1: {
        uint8_t byte = ((const uint8_t *)base)[idx >> 1];
        return dec_e2m1((idx & 1) ? (byte >> 4) : (byte & 0xf));
    }
    case ORC_E8M0:
        return dec_e8m0(((const uint8_t *)base)[idx]);
    case ORC_E5M2:
        return dec_e5m2(((const uint8_t *)base)[idx]);
    case ORC_E2M3:
        return dec_e2m3(fp6_code((const uint8_t *)base, idx));
    case ORC_E3M2:
        return dec_e3m2(fp6_code((const uint8_t *)base, idx));
    }
    return NAN;
}

static int64_t load_int(const void *base, int32_t type, int64_t idx)
{
    if (type == ORC_I8)
        return ((const int8_t *)base)[idx];
    if (type == ORC_I32) {
        int32_t v;
        memcpy(&v, (const char *)base + 4 * idx, 4);
        return v;
    }
    return 0;
}

/* Public decoder, so that tests can pin each format on every code. */
int oracle_decode(int32_t type, const void *src, int64_t count, double *out)
{
    if (type < ORC_F32 || type > ORC_E3M2 || type == 8)
        return -1;
    for (int64_t t = 0; t < count; ++t)
        out[t] = load_real(src, type, t);
    return 0;
}

/* ---------------------------------------------------------------- indexing */

static int64_t a_index(const oracle_problem *p, int64_t i, int64_t q)
{
    return p->op_a == 0 ? i + q * p->lda : q + i * p->lda;
}

static int64_t b_index(const oracle_problem *p, int64_t q, int64_t j)
{
    return p->op_b == 0 ? q + j * p->ldb : j + q * p->ldb;
}

/* ---------------------------------------------------------------- epilogue */

static double activate(int32_t act, double t)
{
    if (act == ORC_ACT_RELU)
        return t > 0.0 ? t : 0.0;
    if (act == ORC_ACT_GELU)
        return 0.5 * t * (1.0 + erf(t / sqrt(2.0))); /* erf form of GELU */
    return t;
}

static int is_integer_path(const oracle_problem *p)
{
    return p->type_a == ORC_I8 && p->type_b == ORC_I8;
}

/* One output element, floating-point path. */
static double element_real(const oracle_problem *p, int64_t i, int64_t j)
{
    double acc = 0.0;
    for (int64_t q = 0; q < p->k; ++q) {
        double a = load_real(p->a, p->type_a, a_index(p, i, q));
        double b = load_real(p->b, p->type_b, b_index(p, q, j));
        if (p->sfa)
            a *= dec_e8m0(p->sfa[i * p->ld_sfa + q / p->block]);
        if (p->sfb)
            b *= dec_e8m0(p->sfb[j * p->ld_sfb + q / p->block]);
        acc += a * b;
    }
    /* Per-tensor scales multiply the finished sum (one rounding). */
    double t = p->alpha * (p->a_scale * p->b_scale * acc);
    if (p->beta != 0.0)
        t += p->beta * load_real(p->c, p->type_c, i + j * p->ldc);
    if (p->bias)
        t += load_real(p->bias, p->type_bias, i);
    return activate(p->act, t);
}

/* One output element, integer path: exact in int64. */
static int64_t element_int(const oracle_problem *p, int64_t i, int64_t j)
{
    int64_t acc = 0;
    for (int64_t q = 0; q < p->k; ++q)
        acc += load_int(p->a, ORC_I8, a_index(p, i, q)) * load_int(p->b, ORC_I8, b_index(p, q, j));
    int64_t t = (int64_t)p->alpha * acc;
    if (p->beta != 0.0)
        t += (int64_t)p->beta * load_int(p->c, p->type_c, i + j * p->ldc);
    if (p->bias)
        t += load_int(p->bias, p->type_bias, i);
    if (p->act == ORC_ACT_RELU && t < 0)
        t = 0;
    return t;
}

/*
 * Evaluate `count` output elements (rows[t], cols[t]).  Floating results go
 * to out_real, integer results (int8 x int8) to out_int; the other pointer
 * may be NULL.  nthreads <= 0 means "all OpenMP threads".  Returns 0, or -1
 * on a request outside the problem.
 */
int oracle_gemm_elements(const oracle_problem *p, int64_t count, const int64_t *rows,
                         const int64_t *cols, double *out_real, int64_t *out_int, int nthreads)
{
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= p->m || cols[t] < 0 || cols[t] >= p->n)
            return -1;
    int integer = is_integer_path(p);
    if ((integer && !out_int) || (!integer && !out_real))
        return -1;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
#endif
    for (int64_t t = 0; t < count; ++t) {
        if (integer)
            out_int[t] = element_int(p, rows[t], cols[t]);
        else
            out_real[t] = element_real(p, rows[t], cols[t]);
    }
    (void)nthreads;
    return 0;
}

/* ------------------------------------------------------- MX output blocks */

/*
 * OCP MX quantization of one block of values (the output side of a
 * block-scaled GEMM: "Technical Documentation: NVIDIA/cutlass", "Blackwell
 * SM100 GEMMs", "Building a Block Scaled Kernel", where the epilogue writes
 * elements plus one scale factor per SFDVectorSize outputs; the rule that
 * turns a block into a scale and elements is the OCP MX format's, which the
 * pages' block-scaled type table points to):
 *
 *   amax = max |v|;  X = floor(log2(amax)) - emax   (emax: the element
 *   format's largest exponent: 2 for E2M1, 8 for E4M3, 15 for E5M2),
 *   clamped to [-127, 127];  scale code = X + 127 (E8M0);
 *   element = the representable value nearest to v / 2^X, ties to the even
 *   code, magnitudes above the largest finite value clamped to it.
 *   A block of zeros gets scale code 0 and zero elements.  Every element
 *   keeps the sign of its value, also when it rounds to zero.
 *
 * fmt is ORC_E2M1, ORC_E4M3 or ORC_E5M2; codes[t] receives element t's code
 * (4 bits for E2M1, sign in bit 3; 8 bits otherwise).  Returns 0, or -1 for
 * an unknown format or count outside 1..32.
 */
int oracle_mx_quantize(int32_t fmt, const double *vals, int64_t count, uint8_t *codes, uint8_t *scale)
{
    int emax, ncodes, sign_bit;
    if (fmt == ORC_E2M1) {
        emax = 2; ncodes = 8; sign_bit = 3;
    } else if (fmt == ORC_E4M3) {
        emax = 8; ncodes = 127; sign_bit = 7; /* 0x7f is NaN */
    } else if (fmt == ORC_E5M2) {
        emax = 15; ncodes = 124; sign_bit = 7; /* 0x7c.. are Inf/NaN */
    } else {
        return -1;
    }
    if (count < 1 || count > 32)
        return -1;
    double amax = 0.0;
    for (int64_t t = 0; t < count; ++t)
        if (fabs(vals[t]) > amax)
            amax = fabs(vals[t]);
    if (amax == 0.0) {
        *scale = 0;
        for (int64_t t = 0; t < count; ++t)
            codes[t] = (uint8_t)(signbit(vals[t]) ? (1 << sign_bit) : 0);
        return 0;
    }
    int x = (int)floor(log2(amax)) - emax;
    /* log2 of an exact power of two is exact; guard the floor against a
     * result just below an integer for values just below a power of two */
    if (ldexp(1.0, x + emax + 1) <= amax)
        x += 1;
    else if (ldexp(1.0, x + emax) > amax)
        x -= 1;
    if (x < -127)
        x = -127;
    if (x > 127)
        x = 127;
    *scale = (uint8_t)(x + 127);
    for (int64_t t = 0; t < count; ++t) {
        double a = fabs(vals[t]) / ldexp(1.0, x);
        /* nearest non-negative code by magnitude; the codes 0 .. ncodes-1
         * are in increasing order of value, and ncodes-1 is the largest
         * finite one, which every larger magnitude clamps to */
        int best = ncodes - 1;
        double top = fmt == ORC_E2M1 ? dec_e2m1((unsigned)best) : (fmt == ORC_E4M3 ? dec_e4m3((uint8_t)best)
                                                                                   : dec_e5m2((uint8_t)best));
        double best_err = INFINITY;
        for (int c = 0; c < ncodes && a < top; ++c) {
            double v = fmt == ORC_E2M1 ? dec_e2m1((unsigned)c) : (fmt == ORC_E4M3 ? dec_e4m3((uint8_t)c)
                                                                                  : dec_e5m2((uint8_t)c));
            double err = fabs(v - a);
            if (err < best_err || (err == best_err && (c & 1) == 0)) {
                best = c;
                best_err = err;
            }
        }
        /* the sign is kept, also when the magnitude rounds to zero */
        codes[t] = (uint8_t)(best | (signbit(vals[t]) ? (1 << sign_bit) : 0));
    }
    return 0;
}

/* Number of threads an OpenMP region would use here (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
