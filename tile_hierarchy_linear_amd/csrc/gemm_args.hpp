// gemm_args.hpp -- kernel arguments and codes shared by the GEMM kernels and
// the host dispatch (no device code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace thl {

// Operand families (one MFMA instruction each).
// FAM_MX8: e4m3 elements with one E8M0 scale per 32 K-elements (MXFP8);
// FAM_MX8_E5M2 the same with e5m2 elements, FAM_MX8_E4E5 / FAM_MX8_E5E4 with
// e4m3 A and e5m2 B and the other way round;
// FAM_E4E5 / FAM_E5E4: e4m3 A with e5m2 B, and the other way round.
enum Family {
  FAM_F16 = 0, FAM_BF16 = 1, FAM_I8 = 2, FAM_FP8 = 3, FAM_FP4 = 4, FAM_E5M2 = 5, FAM_MX8 = 6,
  FAM_E4E5 = 7, FAM_E5E4 = 8, FAM_MX8_E5M2 = 9, FAM_MX8_E4E5 = 10, FAM_MX8_E5E4 = 11
};

// Element-type codes, equal to the public thl_dtype values.
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3, DT_I32 = 4 };
enum : int { EPI_BIAS = 1, EPI_RELU = 2, EPI_GELU = 4 };
// Set by the host, not part of the public flags: D (and C when beta != 0, and
// bias) can be moved as aligned 16-byte vectors along M, C is 16-bit, and a
// 256-column panel of C or D spans less than 2 GiB.
enum : int { EPI_VEC = 8 };

// One problem of a grouped launch, as the caller's device array holds it
// (the same layout as the public thl_group_problem).
struct GroupProblem {
  int64_t m, n, k;
  const void* a;
  int64_t lda;  // elements
  const void* b;
  int64_t ldb;
  const void* c;
  int64_t ldc;
  void* d;
  int64_t ldd;
  const void* bias;
  const uint8_t* sfa;
  int64_t ld_sfa;
  const uint8_t* sfb;
  int64_t ld_sfb;
};

struct GemmArgs {
  const uint8_t* a;  // A as stored: leading dimension lda_bytes
  const uint8_t* b;  // B as stored: leading dimension ldb_bytes
  const void* c;
  void* d;
  const void* bias;
  const uint8_t* sfa;  // fp4: E8M0 scales, row i block kb at sfa[i*ld_sfa + kb]
  const uint8_t* sfb;
  int64_t lda_bytes, ldb_bytes;
  int64_t ldc, ldd;  // elements
  int64_t ld_sfa, ld_sfb;
  int32_t m, n, k;  // k in elements
  int32_t kbytes;   // bytes of K per operand row
  int32_t tiles_m, tiles_n, group_m;
  int32_t xcd_local;  // a multiple of 8 problems: each problem's workgroups share one XCD
  float alpha, beta;  // alpha already holds the per-tensor fp8 scales
  int32_t flags;      // EPI_* bits
  int32_t c_type, d_type, bias_type;
  // Batched problems: problem z's arrays (grid column blockIdx.x of the
  // tiled kernels, row blockIdx.y of the small-M kernel) lie z times these
  // many bytes further (all zero for a single problem).
  int64_t bs_a, bs_b, bs_c, bs_d, bs_bias, bs_sfa, bs_sfb;
  // Grouped problems: grid column blockIdx.x computes group[blockIdx.x] (sizes,
  // pointers and leading dimensions replace the fields above); operand
  // elements are elem_bits_a / elem_bits_b bits wide.  NULL otherwise.
  const GroupProblem* group;
  int32_t elem_bits_a, elem_bits_b;
  // Split K across workgroups: `splits` units per tile (1: none), each over
  // `ksteps` 64-byte K-steps from its split's first, writing its partial
  // product to D + split * split_stride bytes.
  int32_t splits, ksteps;
  int64_t split_stride;
  // MX output (D in an MX element format with one E8M0 scale per 32
  // consecutive rows of a column): mx_out is MX_* (0: none); SFD(b, j) at
  // sfd[j * ld_sfd + b].
  int32_t mx_out;
  uint8_t* sfd;
  int64_t ld_sfd;
};

// MX output element formats.
enum : int { MX_NONE = 0, MX_E4M3 = 1, MX_E5M2 = 2, MX_E2M1 = 3 };


// Launches one kernel variant on `stream`; returns the launch status.
template <int F, int BM, int BN, int WM, int WN, int LOADW, int STAGES, int OCC, int SCW, bool AK, bool BK, bool MXO>
hipError_t launch_gemm(const GemmArgs& a, dim3 grid, hipStream_t stream);

// Launches the small-M kernel (M <= 16 * MT, K-major A and B; KW wavefronts
// split K), one workgroup per 16 columns of D.
template <int F, int KW, int MT>
hipError_t launch_skinny(const GemmArgs& a, dim3 grid, hipStream_t stream);

}  // namespace thl
