/*
 * thl.h -- C ABI of the MI355X (gfx950) tiled GEMM with a fused epilogue,
 *
 *     D = act(alpha * s_a * s_b * op(A) * op(B) + beta * C + bias)
 *
 * and of the host-side Shape:Stride layout module that generates and checks
 * the kernels' index maps.  Plain C: no C++ or torch types cross it; the only
 * HIP type is the stream, declared as the struct pointer hipStream_t is.
 *
 * Sources of the operation (page titles and sections):
 *  - "CUTLASS" (knowledge-base page), opening section: the fixed BLAS surface
 *    C = alpha*op(A)*op(B) + beta*C, and "Epilogues": bias, activation and
 *    scaling applied in the GEMM's output stage with no second pass over C.
 *  - same page: the device GEMM call takes {m,n,k}, {A,lda}, {B,ldb},
 *    {C,ldc}, {D,ldd}, {alpha,beta} and returns a status; "Technical
 *    Documentation: NVIDIA/cutlass", "Launching a GEMM kernel in CUDA": D may
 *    be the same tensor as C.
 *  - same document, "CUTLASS Library": the library picks the first kernel
 *    whose data types, layouts and alignment fit the problem.
 *  - same document, "Blackwell SM100 GEMMs": T = row-major, N = column-major
 *    ("Layouts, Tensor Alignment Requirements"); block-scaled GEMM
 *    D_ij = C_ij + sum_k (A_ik * SFA_{i,k/32}) * (B_jk * SFB_{j,k/32})
 *    ("Block Scaled GEMMs"); element formats e4m3, e2m1, ue8m0 and the
 *    OCP mx types with 32-element scale vectors (the two format tables).
 *  - "CuTe's layout algebra": every layout operation below.
 */
#ifndef THL_H_
#define THL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t*`; NULL = the default stream */

typedef enum {
  THL_OK = 0,
  THL_ERR_INVALID = -1,     /* bad dimension, leading dimension, pointer, overlap or argument */
  THL_ERR_UNSUPPORTED = -2, /* a dtype / op / epilogue / scale combination that is not built */
  THL_ERR_MISALIGNED = -3,  /* a pointer or leading dimension breaks every kernel's alignment */
  THL_ERR_HIP = -4,         /* the HIP runtime reported an error while launching */
  THL_ERR_UNDEFINED = -5,   /* layout algebra: the operation is undefined (divisibility, overlap) */
  THL_ERR_SCRATCH = -6      /* thl_gemm_noalloc: the call needs more than its static scratch */
} thl_status;

/* op(X): N = X as stored, T = its transpose (BLAS convention). */
typedef enum { THL_OP_N = 0, THL_OP_T = 1 } thl_op;

typedef enum {
  THL_F32 = 0,
  THL_F16 = 1,
  THL_BF16 = 2,
  THL_I8 = 3,
  THL_I32 = 4,
  THL_E4M3 = 5,   /* OCP fp8 E4M3 ("fn": bias 7, no infinities, S.1111.111 NaN, max 448) */
  THL_E2M1X2 = 6, /* OCP fp4 E2M1, two per byte along the contiguous dimension, even element low nibble */
  THL_E8M0 = 7,   /* OCP E8M0 scale: 2^(code-127), 0xff NaN */
  THL_NONE = 8,   /* "no such operand" (bias dtype when there is no bias) */
  THL_E5M2 = 9,   /* OCP fp8 E5M2 (bias 15, IEEE-style: S.11111.00 infinity, S.11111.xx NaN, max 57344) */
  THL_E2M3 = 10,  /* OCP fp6 E2M3 (bias 1, all codes finite, max 7.5), bit-packed along the contiguous
                     dimension: element t in bits 6t .. 6t+5 of the little-endian bit stream (four in
                     three bytes) */
  THL_E3M2 = 11   /* OCP fp6 E3M2 (bias 3, all codes finite, max 28), packed as THL_E2M3 */
} thl_dtype;

typedef struct {
  thl_dtype a, b; /* operand formats: a == b (F16, BF16, I8), or any two of E4M3, E5M2, E2M3,
                     E3M2, E2M1X2 (the 8-, 6- and 4-bit float formats, mixed freely) */
  thl_dtype c;    /* format of C: F32, F16 or BF16 for float paths, I32 for the int8 path */
  thl_dtype d;    /* format of D: F32, F16 or BF16 (float paths), I32 (int8 path) */
  thl_dtype bias; /* format of the bias vector: F32, F16, BF16, or I32 (int8 path) */
  thl_dtype acc;  /* accumulation: F32 for float paths, I32 for int8 */
} thl_dtypes;

/* Epilogue flags: RELU and GELU exclusive.  Order: act(alpha*acc + beta*C + bias).
 * GELU is the erf form 0.5*x*(1+erf(x/sqrt 2)). */
enum { THL_EPI_NONE = 0, THL_EPI_BIAS = 1, THL_EPI_RELU = 2, THL_EPI_GELU = 4 };

typedef struct {
  unsigned flags;   /* THL_EPI_* bits */
  const void* bias; /* device pointer, length m (bias[i] is added to row i), when THL_EPI_BIAS */
  uint8_t* sfd;     /* MX output (D in E2M1X2, E4M3 or E5M2): the generated E8M0 scales,
                       SFD(b, j) for rows 32b .. 32b+31 of column j at sfd[j*ld_sfd + b], device;
                       unused otherwise */
  int64_t ld_sfd;   /* >= ceil(m/32) */
} thl_epilogue;

typedef struct {
  float a_scale, b_scale; /* per-tensor scales (host values), used for E4M3 and E5M2 (also mixed and
                             MXFP8); ignored (taken as 1) for the other formats */
  const uint8_t* sfa;     /* E8M0 block scales of A for the MX formats (8-, 6- or 4-bit elements, with
                             sfb): SFA(i,kb) for row i of op(A) and K-elements 32kb .. 32kb+31 at
                             sfa[i*ld_sfa + kb], whatever A's storage, device, 16-byte aligned; NULL
                             for plain formats */
  int64_t ld_sfa;         /* >= k/32 and a multiple of 16 */
  const uint8_t* sfb;     /* SFB(j,kb) at sfb[j*ld_sfb + kb], device, 16-byte aligned; as sfa */
  int64_t ld_sfb;         /* >= k/32 and a multiple of 16 */
} thl_scales;

/*
 * thl_gemm -- D = act(alpha * s_a * s_b * op(A) * op(B) + beta * C + bias[i]).
 *
 * Shapes: op(A) is m x k, op(B) is k x n, C and D are m x n.  Storage is BLAS
 * column-major with leading dimensions in elements:
 *   opA = N: A(i,p) at A[i + p*lda], lda >= max(1,m);   opA = T: at A[p + i*lda], lda >= max(1,k)
 *   opB = N: B(p,j) at B[p + j*ldb], ldb >= max(1,k);   opB = T: at B[j + p*ldb], ldb >= max(1,n)
 *   C(i,j) at C[i + j*ldc], ldc >= max(1,m);  D(i,j) at D[i + j*ldd], ldd >= max(1,m).
 * For E2M1X2 the leading dimension counts fp4 elements and must be even; for
 * E2M3 and E3M2 it counts fp6 elements and must be a multiple of 4 (so that
 * every stored line starts on a whole byte); batch strides likewise.
 *
 * Built combinations (first fitting kernel is launched):
 *   F16 or BF16 operands, opA/opB in {N,T}: F32 accumulate; C, D in F32/F16/BF16.
 *     An operand whose stored lines (rows along K, or k-lines along M or N)
 *     are not whole 4-byte units (an odd leading dimension, batch stride or
 *     base offset), or, with D of 2^23 elements or more, not whole 16-byte
 *     units, is first copied by the conversion pass below into a workspace
 *     at a pitch of whole 64-byte units, in the same layout (variant name
 *     suffix "+cvt_a", "+cvt_b" or "+cvt_ab"); not while THL_FORCE_VARIANT
 *     is set.
 *   I8 operands, opA = T, opB = N: I32 accumulate, C and D I32, bias I32;
 *     alpha must be 1 and beta 0 or 1 (the integer epilogue is exact, in int32).
 *   E4M3 operands, opA = T, opB = N: F32 accumulate, s_a, s_b = scales->a_scale,
 *     b_scale folded with alpha into one fp32 factor.
 *   E5M2 operands (both), opA = T, opB = N: as E4M3.
 *   E4M3 A with E5M2 B, or E5M2 A with E4M3 B, opA = T, opB = N: as E4M3.
 *   fp8 operands (E4M3, E5M2, or one of each) with scales->sfa and
 *     scales->sfb given (MX fp8), opA = T, opB = N, k % 32 == 0: as E2M1X2's
 *     block scales (on top of the per-tensor scales), with the same scale-row
 *     rules.
 *   E2M1X2 operands, opA = T, opB = N, k % 32 == 0: F32 accumulate, element
 *     (i,p) of A multiplied by 2^(SFA(i, p/32) - 127), likewise B with SFB(j, p/32);
 *     scale rows 16-byte aligned (THL_ERR_MISALIGNED otherwise).
 *   Every other layout and pairing of the 8-, 6- and 4-bit formats ("Technical
 *   Documentation: NVIDIA/cutlass", "Layouts, Tensor Alignment Requirements to
 *   Target tcgen05.mma Instructions", Tables 2 and 3: TN, NN, NT, TT, dense or
 *   with E8M0 block scales per 32 K-elements), and I8 in NN, NT, TT: each
 *   operand the tiled kernels cannot stage directly (stored along M or N,
 *   6-bit, or 4-bit beside another format or without block scales) is first
 *   rewritten by a conversion pass into a workspace as K-major rows (variant
 *   name suffix "+cvt_a", "+cvt_b" or "+cvt_ab"): 8-bit formats as they are,
 *   E2M1X2 as E2M1X2 when both operands are block-scaled fp4, and E2M1X2, E2M3
 *   and E3M2 otherwise widened to E4M3, which holds each of their values
 *   exactly; then the TN kernels above run.  K-major 8- and 4-bit rows are
 *   rewritten too (as they are, into 64-byte rows) when they are not whole
 *   4-byte units (no kernel reads them), or not whole 16-byte units and D
 *   has 2^23 elements or more (the 16-byte kernels then win by far more than
 *   the pass costs); not while THL_FORCE_VARIANT is set.  Block scales, when given (both
 *   sfa and sfb, k % 32 == 0), apply per logical row and 32 K-elements
 *   whatever the storage; the per-tensor scales apply to E4M3 and E5M2
 *   operands only.  The workspace is
 *   taken from a stream-ordered pool (THL_ERR_HIP if none can be had) and
 *   returned after the launch; thl_gemm_noalloc takes it from its static
 *   scratch (THL_ERR_SCRATCH when it does not fit).  The pass costs one read
 *   of the operand and one write of its K-major copy (HBM-bound); 6-bit and
 *   widened 4-bit operands then run at the fp8 MFMA rate.  Grouped launches
 *   take only what the kernels stage directly (THL_ERR_UNSUPPORTED otherwise).
 * With m <= 64, k > 0, opA = T and opB = N (any operand family but MXFP8), A and B
 * 16-byte aligned with leading dimensions of whole 16-byte units, the small-M
 * kernel runs (variants "<family>_tn_skinny{16,32,64}_k4", the first whose
 * rows cover m): it streams B once from memory and sums K in a fixed order,
 * so results do not depend on timing.
 * It reads each scale row (E2M1X2) in 8-byte units up to its next 16-byte
 * boundary, as the tiled kernels read it in 16-byte groups.
 *
 * Split K: when a single problem's tiles fill at most a quarter of the
 * device's resident workgroups (128x128 tiles; F16, BF16, I8 and the
 * unscaled fp8 families) and K spans at least 128 steps of 64 bytes, the K
 * range of each tile is split over 2 to 16 workgroups.  Each split writes its
 * partial product (fp32, or int32 for I8) to a matrix of its own, and a
 * second kernel adds the splits' matrices in split order 0, 1, 2, ... (so
 * results do not depend on timing) and applies the epilogue.  The matrices,
 * splits * round_up(m, 4) * n * 4 bytes, come from a stream-ordered memory
 * pool the library creates once per device; they are taken and returned on
 * `stream` around the two kernels.  If the pool cannot provide them the
 * problem runs unsplit.  thl_last_splits reports what ran.
 *
 * Ownership: A, B, C, D, bias, sfa, sfb are device pointers owned by the
 * caller; apart from the split-K workspace above the library allocates
 * nothing, and it keeps no pointer after return.  alpha, beta and the
 * per-tensor scales are host values.
 *
 * MX output ("Technical Documentation: NVIDIA/cutlass", "Building a Block
 * Scaled Kernel": the epilogue writes elements plus one scale factor per
 * block of outputs, blocks along D's contiguous dimension): with the float
 * operand families, dtypes->d may be E2M1X2 (two codes a byte along M, the
 * even row in the low nibble, ldd even), E4M3 or E5M2.  Each run of 32
 * consecutive rows of a column of act(alpha*acc + beta*C + bias), computed in
 * fp32 (the last run of a column may be shorter), becomes one block by the
 * OCP MX rule: scale X = floor(log2 max|v|) - emax (2 for E2M1, 8 for E4M3,
 * 15 for E5M2), clamped to [-127, 127], stored as the E8M0 code X + 127 in
 * epilogue->sfd; elements v / 2^X rounded to nearest even in the element
 * format, magnitudes past its largest finite value clamped to it, signs kept;
 * a block of zeros gets scale code 0.  The tiled kernels' general epilogue
 * writes it (no small-M kernel, no split K), built with 16-byte operand
 * loads only: operand lines that are not whole 16-byte units (base or
 * leading dimension) are first re-pitched by the conversion pass (fp16,
 * bf16 in their own layout; 8- and 4-bit as K-major rows), whatever the
 * size; single problems only (batched and grouped
 * launches return THL_ERR_UNSUPPORTED); sfd must not overlap any other array
 * (THL_ERR_INVALID, as a NULL sfd or a short ld_sfd is).
 *
 * Block scales: sfa or sfb given with F16, BF16 or I8 operands is
 * THL_ERR_UNSUPPORTED.  8-, 6- and 4-bit operands with either array given are
 * MX (MXFP8, MXFP6, MXFP4 or a mix); without either they are plain (dense)
 * formats.  Both arrays are then required (THL_ERR_INVALID otherwise)
 * whenever m > 0, n > 0 and k > 0.
 *
 * Semantics: beta == 0 means C is not read (it may be NULL and may hold NaN).
 * D may alias C exactly (same pointer, ldc == ldd, c and d the same format);
 * any other overlap of D with A, B, C, bias or the scales is THL_ERR_INVALID.
 * m == 0 or n == 0 returns THL_OK with no launch; k == 0 gives
 * D = act(beta*C + bias).  m, n, k and every leading dimension above
 * INT32_MAX, and byte leading dimensions of A or B above 2^23, return
 * THL_ERR_UNSUPPORTED.
 *
 * Errors: every check runs before any HIP call; on an error nothing is
 * enqueued and D is untouched.  The call is asynchronous: it returns once
 * the kernel is enqueued on `stream`, and faults during execution surface at
 * the caller's next synchronisation on that stream.  Reentrant; thread-safe.
 */
thl_status thl_gemm(int64_t m, int64_t n, int64_t k,
                    const void* A, int64_t lda, thl_op opA,
                    const void* B, int64_t ldb, thl_op opB,
                    const void* C, int64_t ldc,
                    void* D, int64_t ldd,
                    float alpha, float beta,
                    const thl_dtypes* dtypes, const thl_epilogue* epilogue,
                    const thl_scales* scales, struct ihipStream_t* stream);

/*
 * thl_gemm_noalloc -- thl_gemm for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, rules and results as thl_gemm; it calls
 * no allocating routine.  Where thl_gemm would split K, the partial matrices
 * go to a static device array of the library (40 MiB, one per GPU, held
 * until the process ends) instead of a pool allocation.  Its address is read
 * once per device, with that device current, at the first call on it.
 * Nothing in the array needs to start at any value: each call writes every
 * partial element it reads.
 * Limit: a call whose split needs more than 40 MiB returns THL_ERR_SCRATCH
 * with nothing enqueued (the splits thl_gemm chooses by itself always fit;
 * only a split count forced through THL_FORCE_SPLITS can exceed it).
 * Concurrency: every call on one GPU uses that GPU's one array, so calls that
 * overlap in time on that GPU (on different streams, or from different
 * threads) race; calls ordered on one stream do not.
 */
thl_status thl_gemm_noalloc(int64_t m, int64_t n, int64_t k,
                            const void* A, int64_t lda, thl_op opA,
                            const void* B, int64_t ldb, thl_op opB,
                            const void* C, int64_t ldc,
                            void* D, int64_t ldd,
                            float alpha, float beta,
                            const thl_dtypes* dtypes, const thl_epilogue* epilogue,
                            const thl_scales* scales, struct ihipStream_t* stream);

/*
 * thl_gemm_batched -- `batch` independent problems of one shape in one launch
 * (the batched GEMM, "L mode", of the "CUTLASS" knowledge-base page and of
 * "Technical Documentation: NVIDIA/cutlass"):
 *   D_z = act(alpha*s_a*s_b*op(A_z)*op(B_z) + beta*C_z + bias_z),  z = 0 .. batch-1,
 * with X_z = X + z*stride_x for X in A, B, C, D, bias (strides in elements of
 * each array's format; E2M1X2 strides count fp4 elements and must be even)
 * and SFA_z = sfa + z*stride_sfa, SFB_z likewise (in bytes).  Every other
 * argument means what it means for thl_gemm and applies to every problem;
 * the same kernel variant runs all of them.  A stride of 0 shares that array
 * between problems (not allowed for D when batch > 1).
 * Extra rules: batch >= 0 (0 returns THL_OK with no launch), batch <= 65535
 * and strides <= 2^40 (else THL_ERR_UNSUPPORTED); strides >= 0 (else
 * THL_ERR_INVALID); with
 * batch > 1, stride_d >= (n-1)*ldd + m so that no two D matrices overlap.
 * Overlap checks take each array's whole span over the batch: D may alias C
 * exactly (also stride_c == stride_d) and may not otherwise overlap the span
 * of A, B, C, bias or the scales, even where the problems would interleave
 * without sharing bytes.  Alignment rules apply to every problem's base
 * (the strides in bytes keep the first base's alignment class).
 */
thl_status thl_gemm_batched(int64_t batch, int64_t m, int64_t n, int64_t k,
                            const void* A, int64_t lda, int64_t stride_a, thl_op opA,
                            const void* B, int64_t ldb, int64_t stride_b, thl_op opB,
                            const void* C, int64_t ldc, int64_t stride_c,
                            void* D, int64_t ldd, int64_t stride_d,
                            float alpha, float beta,
                            const thl_dtypes* dtypes, const thl_epilogue* epilogue, int64_t stride_bias,
                            const thl_scales* scales, int64_t stride_sfa, int64_t stride_sfb,
                            struct ihipStream_t* stream);

/*
 * thl_gemm_grouped -- `count` independent problems of different shapes in one
 * launch (the grouped GEMM of "What's New in CUTLASS 4.8", "CUTLASS Operator
 * API": per-problem sizes, pointers and leading dimensions, as its
 * IndexPtrGroupedGemmArguments carry them):
 *   D_z = act(alpha*s_a*s_b*op(A_z)*op(B_z) + beta*C_z + bias_z),  z = 0 .. count-1,
 * with problem z's m, n, k, arrays and leading dimensions in problems[z].
 * Formats, opA/opB, alpha, beta, the activation flags and the per-tensor
 * scales are one set for the whole group; epilogue->bias is ignored (each
 * problem brings its bias in problems[z].bias, read when THL_EPI_BIAS is
 * set).  Every problem follows the rules of thl_gemm (leading dimensions,
 * alignment, block scales, C == D aliasing), and in addition no problem's D
 * may overlap another problem's D or any array another problem reads.  The
 * problems with outputs (m > 0 and n > 0) must resolve to one operand
 * family: block scales on all of them or on none (THL_ERR_INVALID
 * otherwise); every problem's operands must suit one kernel variant.
 *
 *   problems      host array of `count` descriptors: validated here, and
 *                 used to choose the kernel and the grid.
 *   problems_dev  device array holding the same `count` descriptors (the
 *                 kernel reads each problem's sizes and pointers from it);
 *                 the caller keeps it unchanged until the launch completes.
 *
 * Only what the tiled kernels stage directly is built grouped: operands
 * that thl_gemm would first rewrite (see "Every other layout and pairing"
 * above: 8-bit formats stored along M or N, fp6, fp4 beside another format
 * or without block scales) and MX-format D return THL_ERR_UNSUPPORTED.
 * One kernel variant (the tiled kernels; the small-M kernel is not used)
 * runs every problem; grid row z computes problem z with its share of
 * persistent workgroups.  count == 0, or every problem with m == 0 or
 * n == 0, returns THL_OK with no launch; count above 65535 returns
 * THL_ERR_UNSUPPORTED; a NULL problems_dev with work to do is
 * THL_ERR_INVALID.  Errors as for thl_gemm (nothing is enqueued).
 */
typedef struct {
  int64_t m, n, k;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  const void* C; /* read when beta != 0 */
  int64_t ldc;
  void* D;
  int64_t ldd;
  const void* bias; /* length m, read when THL_EPI_BIAS is set */
  const uint8_t* sfa; /* E8M0 block scales (E2M1X2, MX fp8), as for thl_gemm */
  int64_t ld_sfa;
  const uint8_t* sfb;
  int64_t ld_sfb;
} thl_group_problem;

thl_status thl_gemm_grouped(int64_t count, const thl_group_problem* problems,
                            const thl_group_problem* problems_dev, thl_op opA, thl_op opB,
                            float alpha, float beta, const thl_dtypes* dtypes,
                            const thl_epilogue* epilogue, const thl_scales* scales,
                            struct ihipStream_t* stream);

/* Static text for a status code. */
const char* thl_status_string(int status);

/* Name of the kernel variant the calling thread's last successful thl_gemm
 * launched ("" before any); the storage is thread-local and stays valid until
 * the thread's next thl_gemm call.  "<variant>+cvt_a" (b, ab): the operands
 * named went through the conversion pass first.  "<first>|<rest>": a single
 * problem whose 256x256 tiles would fill at most half of a last round of the
 * device's CUs ran as two launches, the rows of whole rounds on <first> and
 * the remaining rows as a problem of their own on <rest>. */
const char* thl_last_variant(void);

/* Number of K splits (workgroups sharing each output tile) of the calling
 * thread's last successful launch: 1 unless thl_gemm split K (see thl_gemm,
 * "Split K"). */
int thl_last_splits(void);

/* Number of kernel variants built into the library, and the name of each
 * (static strings).  Setting THL_FORCE_VARIANT=<name> in the environment makes
 * thl_gemm launch that variant, or fail with THL_ERR_UNSUPPORTED when it does
 * not fit the problem (tests use it to cover every variant). */
int thl_variant_count(void);
const char* thl_variant_name(int index);

/*
 * thl_kernel_index_map -- evaluate one of the kernels' closed-form index
 * functions on the host, for checking against the layout module.
 *   map     name of the map (thl_kernel_index_map_names lists them)
 *   params  map parameters (e.g. tile counts), may be NULL when none
 *   n       number of points; in[2*t], in[2*t+1] are the two arguments
 *   out     out[2*t], out[2*t+1] receive the two results
 * These are the same `__host__ __device__` functions the kernels call.
 * Returns THL_OK, or THL_ERR_INVALID for an unknown name or bad arguments.
 */
int thl_kernel_index_map(const char* map, const int64_t* params, int64_t n, const int64_t* in, int64_t* out);
/* Comma-separated names of every map thl_kernel_index_map knows (static). */
const char* thl_kernel_index_map_names(void);

/*
 * Layout algebra ("CuTe's layout algebra").  Host only, run-time integers,
 * full simplification.  A layout is text "shape:stride" with nested tuples,
 * e.g. "(4,(2,4)):(2,(1,8))"; a bare shape means the compact column-major
 * layout; underscores are ignored so "_12:_1" parses.  A tiler is one layout
 * per mode, separated by ';' ("2:1;2:1").  Results are written to `out` as
 * NUL-terminated text of at most `cap` bytes.  Each returns THL_OK,
 * THL_ERR_INVALID (parse error, mismatched structure, output too small, index
 * out of range) or THL_ERR_UNDEFINED (the operation is undefined: a shape or
 * stride divisibility condition fails, or the modes overlap).
 */
int thl_layout_coalesce(const char* a, char* out, size_t cap);
/* R = A o B, R(c) = A(B(c)), R has B's shape; b may be a ';' tiler (mode by mode). */
int thl_layout_composition(const char* a, const char* b, char* out, size_t cap);
/* A* such that (A, A*) covers [0, cotarget) exactly once. */
int thl_layout_complement(const char* a, int64_t cotarget, char* out, size_t cap);
/* A o (B, complement(B, size A)); b may be a ';' tiler. */
int thl_layout_logical_divide(const char* a, const char* b, char* out, size_t cap);
/* ((within-tile modes), (tile-index modes)). */
int thl_layout_zipped_divide(const char* a, const char* tiler, char* out, size_t cap);
/* ((within-tile modes), tile-index mode 0, tile-index mode 1, ...). */
int thl_layout_tiled_divide(const char* a, const char* tiler, char* out, size_t cap);
/* (within-tile modes..., tile-index modes...). */
int thl_layout_flat_divide(const char* a, const char* tiler, char* out, size_t cap);
/* The tile with one-dimensional tile index `tile`: its layout, and *offset = index of its origin. */
int thl_layout_local_tile(const char* a, const char* tiler, int64_t tile, int64_t* offset, char* out, size_t cap);
/* Thread `tid`'s values when A is divided by the shape of `threads`: *offset is
 * the index of its within-tile position p (threads(p) == tid); the layout is the tile-index mode. */
int thl_layout_local_partition(const char* a, const char* threads, int64_t tid, int64_t* offset, char* out,
                               size_t cap);
/* out[i] = A(crd[i]) for one-dimensional coordinates. */
int thl_layout_eval(const char* a, const int64_t* crd, int64_t n, int64_t* out);
/* *out = A(coord) for a top-level or nested coordinate written as text, e.g. "(1,(1,2))". */
int thl_layout_eval_coord(const char* a, const char* coord, int64_t* out);
/* size, cosize (largest index + 1) and rank (top-level modes); any pointer may be NULL. */
int thl_layout_info(const char* a, int64_t* size, int64_t* cosize, int64_t* rank);
/* Mode i of A as a layout. */
int thl_layout_mode(const char* a, int64_t i, char* out, size_t cap);
/* out[i] = swz(A(crd[i])) with swz(x) = x ^ (((x >> (m+s)) & (2^b - 1)) << m):
 * the XOR function composed on top of a layout (used for LDS bank spreading). */
int thl_swizzle_eval(int b, int m, int s, const char* a, const int64_t* crd, int64_t n, int64_t* out);

#ifdef __cplusplus
}
#endif

#endif /* THL_H_ */
