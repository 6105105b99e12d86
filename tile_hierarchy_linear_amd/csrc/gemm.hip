// gemm.hip -- the thl_gemm and thl_gemm_batched C ABI: validation, first-fit
// variant selection, launch, and host evaluation of the kernels' index maps.
//
// The operand family follows the dtypes: one per format, the two mixed fp8
// orders, and MXFP8 for E4M3 operands given block scales.  Selection follows
// the page's rule for the library's host API: the first built kernel whose
// data types, layouts and alignment fit the problem ("Technical
// Documentation: NVIDIA/cutlass", "CUTLASS Library"), with two shape rules on
// top.  Problems with at most 64 rows of op(A) first try the small-M kernel,
// which streams B once.  Otherwise the largest tile whose tile count (over
// the whole batch) still fills the 256 compute units is tried first: 256x256
// tiles with one workgroup per CU, then 256x128 with two per CU, then
// 128x128.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "../../include/thl.h"
#include "convert.hpp"
#include "gemm_args.hpp"
#include "index_maps.hpp"

namespace thl {

static_assert(sizeof(GroupProblem) == sizeof(thl_group_problem), "device descriptors are the public ones");
static_assert(offsetof(GroupProblem, ld_sfb) == offsetof(thl_group_problem, ld_sfb), "same layout");

namespace {

using LaunchFn = hipError_t (*)(const GemmArgs&, dim3, hipStream_t);

struct Variant {
  const char* name;
  int family;
  bool a_kmajor, b_kmajor;  // opA == T, opB == N
  int bm, bn, threads, loadw;
  int occ;   // workgroups per CU the kernel is built for
  int tier;  // 0: 256x256, 1: 256x128, 2: 128x128 (the shape rule's preference order);
             // -1: the small-M kernel (M <= bm <= 64), chosen by its own rule
  LaunchFn launch;
  bool mxout = false;  // writes MX-format D (elements plus generated scales); chosen only for such D
};

#define THL_V(FAM, NAME, OPS, AK, BK, BM, BN, LOADW, ST, OCC, TIER)                                       \
  {NAME "_" OPS "_" #BM "x" #BN "_v" #LOADW "_s" #ST "_o" #OCC, FAM, AK, BK, BM, BN, 256, LOADW, OCC, TIER, \
   &launch_gemm<FAM, BM, BN, 2, 2, LOADW, ST, OCC, 16, AK, BK, false>}

// The MX-output variant (must match THL_INST_MXOUT).
#define THL_VMXO(FAM, NAME, OPS, AK, BK)                                                         \
  {NAME "_" OPS "_128x128_v16_s4_o2_mxout", FAM, AK, BK, 128, 128, 256, 16, 2, 2,              \
   &launch_gemm<FAM, 128, 128, 2, 2, 16, 4, 2, 16, AK, BK, true>, true}

// Must list exactly the instantiations of THL_INSTANTIATE_VARIANTS.  Order is
// the first-fit order within a tier: 16-byte copies before 4-byte ones.  The
// 128x128 variant with one workgroup per CU and six stages is taken only for
// a launch whose tiles fit one round of the CUs (choose_variant).
#define THL_VARIANTS(FAM, NAME, OPS, AK, BK)                  \
  THL_V(FAM, NAME, OPS, AK, BK, 256, 256, 16, 4, 1, 0),       \
      THL_V(FAM, NAME, OPS, AK, BK, 256, 128, 16, 3, 2, 1),   \
      THL_V(FAM, NAME, OPS, AK, BK, 128, 128, 16, 6, 1, 2),   \
      THL_V(FAM, NAME, OPS, AK, BK, 128, 128, 16, 4, 2, 2),   \
      THL_V(FAM, NAME, OPS, AK, BK, 128, 128, 4, 4, 2, 2)

// The MX fp8 families (no 256x128 variant: their scale groups of eight
// K-steps need a stage count that divides into them).
#define THL_VMX8(FAM, NAME)                                      \
  THL_V(FAM, NAME, "tn", true, true, 256, 256, 16, 4, 1, 0),     \
      THL_V(FAM, NAME, "tn", true, true, 128, 128, 16, 4, 2, 2), \
      THL_V(FAM, NAME, "tn", true, true, 128, 128, 4, 4, 2, 2)

// The small-M kernel: 16 columns and 16, 32 or 64 rows of D per workgroup, K
// split over 4 wavefronts (the first whose rows cover M is chosen).
#define THL_VS1(FAM, NAME, MT, ROWS) \
  {NAME "_tn_skinny" #ROWS "_k4", FAM, true, true, ROWS, 16, 256, 16, 2, -1, &launch_skinny<FAM, 4, MT>}
#define THL_VS(FAM, NAME) THL_VS1(FAM, NAME, 1, 16), THL_VS1(FAM, NAME, 2, 32), THL_VS1(FAM, NAME, 4, 64)

const Variant kVariants[] = {
    THL_VARIANTS(FAM_BF16, "bf16", "tn", true, true),
    THL_VARIANTS(FAM_BF16, "bf16", "nn", false, true),
    THL_VARIANTS(FAM_BF16, "bf16", "tt", true, false),
    THL_VARIANTS(FAM_BF16, "bf16", "nt", false, false),
    THL_VARIANTS(FAM_F16, "f16", "tn", true, true),
    THL_VARIANTS(FAM_F16, "f16", "nn", false, true),
    THL_VARIANTS(FAM_F16, "f16", "tt", true, false),
    THL_VARIANTS(FAM_F16, "f16", "nt", false, false),
    THL_VARIANTS(FAM_I8, "i8", "tn", true, true),
    THL_VARIANTS(FAM_FP8, "e4m3", "tn", true, true),
    THL_VARIANTS(FAM_E5M2, "e5m2", "tn", true, true),
    THL_VARIANTS(FAM_E4E5, "e4m3e5m2", "tn", true, true),
    THL_VARIANTS(FAM_E5E4, "e5m2e4m3", "tn", true, true),
    THL_V(FAM_FP4, "e2m1", "tn", true, true, 256, 256, 16, 4, 1, 0),
    THL_V(FAM_FP4, "e2m1", "tn", true, true, 128, 128, 16, 4, 2, 2),
    THL_V(FAM_FP4, "e2m1", "tn", true, true, 128, 128, 4, 4, 2, 2),
    THL_VMX8(FAM_MX8, "mxe4m3"),
    THL_VMX8(FAM_MX8_E5M2, "mxe5m2"),
    THL_VMX8(FAM_MX8_E4E5, "mxe4m3e5m2"),
    THL_VMX8(FAM_MX8_E5E4, "mxe5m2e4m3"),
    THL_VMXO(FAM_BF16, "bf16", "tn", true, true),
    THL_VMXO(FAM_BF16, "bf16", "nn", false, true),
    THL_VMXO(FAM_BF16, "bf16", "tt", true, false),
    THL_VMXO(FAM_BF16, "bf16", "nt", false, false),
    THL_VMXO(FAM_F16, "f16", "tn", true, true),
    THL_VMXO(FAM_F16, "f16", "nn", false, true),
    THL_VMXO(FAM_F16, "f16", "tt", true, false),
    THL_VMXO(FAM_F16, "f16", "nt", false, false),
    THL_VMXO(FAM_FP8, "e4m3", "tn", true, true),
    THL_VMXO(FAM_E5M2, "e5m2", "tn", true, true),
    THL_VMXO(FAM_E4E5, "e4m3e5m2", "tn", true, true),
    THL_VMXO(FAM_E5E4, "e5m2e4m3", "tn", true, true),
    THL_VMXO(FAM_MX8, "mxe4m3", "tn", true, true),
    THL_VMXO(FAM_MX8_E5M2, "mxe5m2", "tn", true, true),
    THL_VMXO(FAM_MX8_E4E5, "mxe4m3e5m2", "tn", true, true),
    THL_VMXO(FAM_MX8_E5E4, "mxe5m2e4m3", "tn", true, true),
    THL_VMXO(FAM_FP4, "e2m1", "tn", true, true),
    THL_VS(FAM_BF16, "bf16"),
    THL_VS(FAM_F16, "f16"),
    THL_VS(FAM_I8, "i8"),
    THL_VS(FAM_FP8, "e4m3"),
    THL_VS(FAM_E5M2, "e5m2"),
    THL_VS(FAM_E4E5, "e4m3e5m2"),
    THL_VS(FAM_E5E4, "e5m2e4m3"),
    THL_VS(FAM_FP4, "e2m1"),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

thread_local const char* t_last_variant = "";
thread_local char t_rows_name[256];  // a problem run as two row ranges: "<first>|<rest>"
thread_local int last_splits = 1;

// Compute units of a device, read once per device.
std::atomic<int> g_cu_count[64];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// ---- split K
// With split K each work unit writes its partial product, unscaled, to an
// fp32 (int32) matrix of its own split; splitk_reduce then adds the splits'
// matrices in split order 0, 1, 2, ... and applies the epilogue proper
// (alpha and the per-tensor scales, beta*C, bias, activation, rounding to
// D's format).  thl_gemm draws the matrices per call from a stream-ordered
// pool the library creates once per device (memory stays in the pool
// between calls) and returns them on the stream after the two kernels.

struct ReduceArgs {
  const uint8_t* ws;     // the splits' matrices: column j of split s at ws + s*stride + j*ld_ws*4
  int64_t ld_ws, stride; // elements per column, bytes per split
  int32_t splits, m, n, int_path;
  const void* c;
  int64_t ldc;
  int32_t c_type;
  const void* bias;
  int32_t bias_type;
  void* d;
  int64_t ldd;
  int32_t d_type;
  float alpha, beta;  // alpha holds the per-tensor fp8 scales
  int32_t flags;
};

__device__ __forceinline__ float ld_float(const void* p, int t, int64_t i) {
  if (t == THL_F32) return static_cast<const float*>(p)[i];
  if (t == THL_F16) return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  return static_cast<float>(static_cast<const __bf16*>(p)[i]);
}

__device__ __forceinline__ void st_float(void* p, int t, int64_t i, float v) {
  if (t == THL_F32) {
    static_cast<float*>(p)[i] = v;
  } else if (t == THL_F16) {
    static_cast<_Float16*>(p)[i] = static_cast<_Float16>(v);
  } else {
    static_cast<__bf16*>(p)[i] = static_cast<__bf16>(v);
  }
}

// One thread per 4 rows of a column, consecutive threads down the column.
__global__ void __launch_bounds__(256) splitk_reduce(ReduceArgs r) {
  const int64_t chunks_per_col = (r.m + 3) / 4;
  const int64_t total = chunks_per_col * r.n;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < total;
       q += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t j = q / chunks_per_col, i0 = (q - j * chunks_per_col) * 4;
    const uint8_t* col = r.ws + j * r.ld_ws * 4 + i0 * 4;
    const int rows = r.m - i0 < 4 ? static_cast<int>(r.m - i0) : 4;
    if (r.int_path) {
      int4 acc = *reinterpret_cast<const int4*>(col);
      for (int s = 1; s < r.splits; ++s) {
        const int4 v = *reinterpret_cast<const int4*>(col + s * r.stride);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
      const int sum[4] = {acc.x, acc.y, acc.z, acc.w};
      for (int e = 0; e < rows; ++e) {
        const int64_t i = i0 + e;
        int t = sum[e];
        if (r.beta != 0.0f) t += static_cast<const int*>(r.c)[j * r.ldc + i];
        if (r.flags & THL_EPI_BIAS) t += static_cast<const int*>(r.bias)[i];
        if ((r.flags & THL_EPI_RELU) && t < 0) t = 0;
        static_cast<int*>(r.d)[j * r.ldd + i] = t;
      }
    } else {
      float4 acc = *reinterpret_cast<const float4*>(col);
      for (int s = 1; s < r.splits; ++s) {
        const float4 v = *reinterpret_cast<const float4*>(col + s * r.stride);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
      const float sum[4] = {acc.x, acc.y, acc.z, acc.w};
      for (int e = 0; e < rows; ++e) {
        const int64_t i = i0 + e;
        float t = r.alpha * sum[e];
        if (r.beta != 0.0f) t += r.beta * ld_float(r.c, r.c_type, j * r.ldc + i);
        if (r.flags & THL_EPI_BIAS) t += ld_float(r.bias, r.bias_type, i);
        if (r.flags & THL_EPI_RELU) t = t > 0.0f ? t : 0.0f;
        if (r.flags & THL_EPI_GELU) t = 0.5f * t * (1.0f + erff(t * 0.70710678118654752440f));
        st_float(r.d, r.d_type, j * r.ldd + i, t);
      }
    }
  }
}

std::mutex g_pool_mutex;
hipMemPool_t g_pools[64];

hipMemPool_t pool_for_device(int dev) {
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_pool_mutex);
  if (!g_pools[dev]) {
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) != hipSuccess) return nullptr;
    uint64_t keep = UINT64_MAX;  // keep freed blocks for the next call
    (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    g_pools[dev] = pool;
  }
  return g_pools[dev];
}

int family_of(thl_dtype t) {
  switch (t) {
    case THL_F16:
      return FAM_F16;
    case THL_BF16:
      return FAM_BF16;
    case THL_I8:
      return FAM_I8;
    case THL_E4M3:
      return FAM_FP8;
    case THL_E5M2:
      return FAM_E5M2;
    case THL_E2M1X2:
      return FAM_FP4;
    default:
      return -1;
  }
}

// Bytes of `count` elements of a format (fp4: two per byte, rounded up).
int64_t bytes_of(thl_dtype t, int64_t count) {
  switch (t) {
    case THL_F32:
    case THL_I32:
      return 4 * count;
    case THL_F16:
    case THL_BF16:
      return 2 * count;
    case THL_I8:
    case THL_E4M3:
    case THL_E5M2:
    case THL_E8M0:
      return count;
    case THL_E2M1X2:
      return (count + 1) / 2;
    case THL_E2M3:
    case THL_E3M2:
      return (6 * count + 7) / 8;
    default:
      return 0;
  }
}

// Bits of one element of an operand format.
int bits_of(thl_dtype t) {
  return t == THL_E2M1X2 ? 4 : ((t == THL_E2M3 || t == THL_E3M2) ? 6 : 8 * static_cast<int>(bytes_of(t, 1)));
}

bool is_float_io(thl_dtype t) { return t == THL_F32 || t == THL_F16 || t == THL_BF16; }

// D formats written as MX blocks (elements plus generated E8M0 scales).
int mx_out_of(thl_dtype t) {
  return t == THL_E4M3 ? MX_E4M3 : (t == THL_E5M2 ? MX_E5M2 : (t == THL_E2M1X2 ? MX_E2M1 : MX_NONE));
}
bool is_mx_out(thl_dtype t) { return mx_out_of(t) != MX_NONE; }

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi), empty when lo == hi
};

// Byte range spanned by a column-major r x c matrix with leading dimension ld.
Range matrix_range(const void* p, thl_dtype t, int64_t r, int64_t c, int64_t ld) {
  Range g;
  if (!p || r <= 0 || c <= 0) return g;
  g.lo = reinterpret_cast<uintptr_t>(p);
  g.hi = g.lo + static_cast<uintptr_t>(bytes_of(t, (c - 1) * ld + r));
  return g;
}

bool overlaps(const Range& a, const Range& b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

// Batched problems (L mode): `count` problems whose arrays lie at fixed
// strides, in elements of each array's own format (E8M0 bytes for scales).
struct Batch {
  int64_t count = 1;
  int64_t a = 0, b = 0, c = 0, d = 0, bias = 0, sfa = 0, sfb = 0;
};

// Byte range spanned by `count` r x c matrices `stride` elements apart.
Range batch_range(const void* p, thl_dtype t, int64_t r, int64_t c, int64_t ld, int64_t count, int64_t stride) {
  Range g = matrix_range(p, t, r, c, ld);
  if (g.lo < g.hi && count > 1) g.hi += static_cast<uintptr_t>(bytes_of(t, (count - 1) * stride));
  return g;
}

bool aligned(const void* p, int64_t pitch_bytes, int w) {
  return (reinterpret_cast<uintptr_t>(p) % w) == 0 && (pitch_bytes % w) == 0;
}

// Where a split-K workspace comes from: a stream-ordered pool allocation
// (thl_gemm), or the library's static scratch array (the no-allocation
// entry point).
enum { WS_POOL = 0, WS_STATIC = 1 };

thl_status gemm_impl(const Batch& bt, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda, thl_op opA,
                     const void* B, int64_t ldb, thl_op opB, const void* C, int64_t ldc, void* D, int64_t ldd,
                     float alpha, float beta, const thl_dtypes* dt, const thl_epilogue* epi, const thl_scales* sc,
                     struct ihipStream_t* stream, int ws_mode, int64_t ws_offset = 0);
thl_status grouped_impl(int64_t count, const thl_group_problem* pb, const thl_group_problem* pb_dev, thl_op opA,
                        thl_op opB, float alpha, float beta, const thl_dtypes* dt, const thl_epilogue* epi,
                        const thl_scales* sc, struct ihipStream_t* stream);

}  // namespace
}  // namespace thl

using namespace thl;

extern "C" {

const char* thl_status_string(int s) {
  switch (s) {
    case THL_OK:
      return "THL_OK";
    case THL_ERR_INVALID:
      return "THL_ERR_INVALID: bad dimension, leading dimension, pointer, overlap or argument";
    case THL_ERR_UNSUPPORTED:
      return "THL_ERR_UNSUPPORTED: combination not built";
    case THL_ERR_MISALIGNED:
      return "THL_ERR_MISALIGNED: pointer or leading dimension breaks every kernel's alignment";
    case THL_ERR_HIP:
      return "THL_ERR_HIP: the HIP runtime reported a launch error";
    case THL_ERR_UNDEFINED:
      return "THL_ERR_UNDEFINED: layout operation undefined (divisibility or overlap)";
    case THL_ERR_SCRATCH:
      return "THL_ERR_SCRATCH: the call needs more than the no-allocation entry point's 40 MiB of scratch";
    default:
      return "unknown status";
  }
}

const char* thl_last_variant(void) { return t_last_variant; }

int thl_last_splits(void) { return last_splits; }

int thl_variant_count(void) { return kNumVariants; }

const char* thl_variant_name(int i) { return (i >= 0 && i < kNumVariants) ? kVariants[i].name : nullptr; }

thl_status thl_gemm(int64_t m, int64_t n, int64_t k, const void* A, int64_t lda, thl_op opA, const void* B,
                    int64_t ldb, thl_op opB, const void* C, int64_t ldc, void* D, int64_t ldd, float alpha,
                    float beta, const thl_dtypes* dt, const thl_epilogue* epi, const thl_scales* sc,
                    struct ihipStream_t* stream) {
  return gemm_impl(Batch{}, m, n, k, A, lda, opA, B, ldb, opB, C, ldc, D, ldd, alpha, beta, dt, epi, sc, stream, WS_POOL);
}

thl_status thl_gemm_noalloc(int64_t m, int64_t n, int64_t k, const void* A, int64_t lda, thl_op opA, const void* B,
                            int64_t ldb, thl_op opB, const void* C, int64_t ldc, void* D, int64_t ldd, float alpha,
                            float beta, const thl_dtypes* dt, const thl_epilogue* epi, const thl_scales* sc,
                            struct ihipStream_t* stream) {
  return gemm_impl(Batch{}, m, n, k, A, lda, opA, B, ldb, opB, C, ldc, D, ldd, alpha, beta, dt, epi, sc, stream,
                   WS_STATIC);
}

thl_status thl_gemm_batched(int64_t batch, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda,
                            int64_t stride_a, thl_op opA, const void* B, int64_t ldb, int64_t stride_b, thl_op opB,
                            const void* C, int64_t ldc, int64_t stride_c, void* D, int64_t ldd, int64_t stride_d,
                            float alpha, float beta, const thl_dtypes* dt, const thl_epilogue* epi,
                            int64_t stride_bias, const thl_scales* sc, int64_t stride_sfa, int64_t stride_sfb,
                            struct ihipStream_t* stream) {
  Batch bt;
  bt.count = batch;
  bt.a = stride_a;
  bt.b = stride_b;
  bt.c = stride_c;
  bt.d = stride_d;
  bt.bias = stride_bias;
  bt.sfa = stride_sfa;
  bt.sfb = stride_sfb;
  return gemm_impl(bt, m, n, k, A, lda, opA, B, ldb, opB, C, ldc, D, ldd, alpha, beta, dt, epi, sc, stream, WS_POOL);
}

thl_status thl_gemm_grouped(int64_t count, const thl_group_problem* problems, const thl_group_problem* problems_dev,
                            thl_op opA, thl_op opB, float alpha, float beta, const thl_dtypes* dtypes,
                            const thl_epilogue* epilogue, const thl_scales* scales, struct ihipStream_t* stream) {
  return grouped_impl(count, problems, problems_dev, opA, opB, alpha, beta, dtypes, epilogue, scales, stream);
}

}  // extern "C"

namespace thl {
namespace {

// Everything the validation of one problem establishes: its family, flags,
// byte leading dimensions and scales, and the conditions the variant choice
// and the kernel arguments depend on.
struct Prep {
  int fam = -1;
  bool a_kmajor = false, b_kmajor = false, block_scaled = false, int_path = false, has_bias = false;
  bool small_m = false, work = false, vec = false, rows16 = true;
  int mx_out = MX_NONE;  // D in an MX element format, with generated scales
  unsigned flags = 0;
  int64_t lda_bytes = 0, ldb_bytes = 0, sa_bytes = 0, sb_bytes = 0;
  thl_scales s{1.0f, 1.0f, nullptr, 0, nullptr, 0};
};

// Validate one problem (all of thl_gemm's rules, for `bt.count` problems at
// the batch strides); nothing touches the device.
thl_status prepare(const Batch& bt, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda, thl_op opA,
                   const void* B, int64_t ldb, thl_op opB, const void* C, int64_t ldc, void* D, int64_t ldd,
                   float alpha, float beta, const thl_dtypes* dt, unsigned flags, const void* bias,
                   const thl_scales* sc, const uint8_t* sfd, int64_t ld_sfd, Prep* out) {
  // ---- arguments
  if (!dt || m < 0 || n < 0 || k < 0) return THL_ERR_INVALID;
  if (bt.count < 0 || bt.a < 0 || bt.b < 0 || bt.c < 0 || bt.d < 0 || bt.bias < 0 || bt.sfa < 0 || bt.sfb < 0)
    return THL_ERR_INVALID;
  if (bt.count > 65535) return THL_ERR_UNSUPPORTED;  // one grid row per problem
  // Byte spans below are computed in int64: leading dimensions up to 2^31 and
  // batch strides up to 2^40 elements keep every product in range.
  if (lda > INT32_MAX || ldb > INT32_MAX || ldc > INT32_MAX || ldd > INT32_MAX) return THL_ERR_UNSUPPORTED;
  constexpr int64_t kMaxStride = INT64_C(1) << 40;
  if (bt.a > kMaxStride || bt.b > kMaxStride || bt.c > kMaxStride || bt.d > kMaxStride || bt.bias > kMaxStride ||
      bt.sfa > kMaxStride || bt.sfb > kMaxStride)
    return THL_ERR_UNSUPPORTED;
  if ((opA != THL_OP_N && opA != THL_OP_T) || (opB != THL_OP_N && opB != THL_OP_T)) return THL_ERR_INVALID;
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return THL_ERR_UNSUPPORTED;
  if (flags & ~static_cast<unsigned>(THL_EPI_BIAS | THL_EPI_RELU | THL_EPI_GELU)) return THL_ERR_INVALID;
  if ((flags & THL_EPI_RELU) && (flags & THL_EPI_GELU)) return THL_ERR_INVALID;
  const bool has_bias = (flags & THL_EPI_BIAS) != 0;

  // ---- supported combinations
  // One fp8 format for A and the other for B is the mixed family of that order.
  const int fam0 = family_of(dt->a);
  const bool f8a = dt->a == THL_E4M3 || dt->a == THL_E5M2, f8b = dt->b == THL_E4M3 || dt->b == THL_E5M2;
  const bool mixed = f8a && f8b && dt->a != dt->b;
  // fp8 operands with block-scale arrays are MX fp8 (MXFP8 with E4M3 or E5M2
  // elements, or one of each); both arrays are then required once the
  // problem has outputs and k > 0 (an empty operand may come without one).
  const bool any_sf = sc && (sc->sfa || sc->sfb);
  const bool mx8 = f8a && f8b && any_sf;
  int fam = fam0;
  if (mx8) {
    fam = !mixed ? (dt->a == THL_E4M3 ? FAM_MX8 : FAM_MX8_E5M2) : (dt->a == THL_E4M3 ? FAM_MX8_E4E5 : FAM_MX8_E5E4);
  } else if (mixed) {
    fam = dt->a == THL_E4M3 ? FAM_E4E5 : FAM_E5E4;
  }
  if (fam < 0 || (dt->b != dt->a && !mixed)) return THL_ERR_UNSUPPORTED;
  // Block scales come with E2M1 and fp8 operands only.
  if (any_sf && fam != FAM_FP4 && !mx8) return THL_ERR_UNSUPPORTED;
  const bool block_scaled = fam == FAM_FP4 || mx8;
  const bool int_path = fam == FAM_I8;
  if (int_path) {
    if (dt->acc != THL_I32 || dt->d != THL_I32) return THL_ERR_UNSUPPORTED;
    if (beta != 0.0f && dt->c != THL_I32) return THL_ERR_UNSUPPORTED;
    if (has_bias && dt->bias != THL_I32) return THL_ERR_UNSUPPORTED;
    if (alpha != 1.0f || (beta != 0.0f && beta != 1.0f)) return THL_ERR_UNSUPPORTED;
    if (flags & THL_EPI_GELU) return THL_ERR_UNSUPPORTED;
  } else {
    if (dt->acc != THL_F32 || !(is_float_io(dt->d) || is_mx_out(dt->d))) return THL_ERR_UNSUPPORTED;
    if (beta != 0.0f && !is_float_io(dt->c)) return THL_ERR_UNSUPPORTED;
    if (has_bias && !is_float_io(dt->bias)) return THL_ERR_UNSUPPORTED;
  }
  // MX output: D in E2M1 (two a byte along M), E4M3 or E5M2 with one E8M0
  // scale per 32 consecutive rows of a column, for one problem at a time.
  const int mx_out = int_path ? MX_NONE : mx_out_of(dt->d);
  if (mx_out != MX_NONE && bt.count > 1) return THL_ERR_UNSUPPORTED;
  // 8- and 4-bit operands: K-major only (op(A) rows, op(B) columns contiguous along K).
  const bool a_kmajor = opA == THL_OP_T, b_kmajor = opB == THL_OP_N;
  if (fam != FAM_BF16 && fam != FAM_F16 && (!a_kmajor || !b_kmajor)) return THL_ERR_UNSUPPORTED;
  if (block_scaled && (k % 32 != 0)) return THL_ERR_UNSUPPORTED;

  // ---- leading dimensions and pointers
  const int64_t rows_a = (opA == THL_OP_N) ? m : k, cols_a = (opA == THL_OP_N) ? k : m;
  const int64_t rows_b = (opB == THL_OP_N) ? k : n, cols_b = (opB == THL_OP_N) ? n : k;
  if (lda < (rows_a > 1 ? rows_a : 1) || ldb < (rows_b > 1 ? rows_b : 1)) return THL_ERR_INVALID;
  if (ldd < (m > 1 ? m : 1)) return THL_ERR_INVALID;
  if (beta != 0.0f && ldc < (m > 1 ? m : 1)) return THL_ERR_INVALID;
  if (fam == FAM_FP4 && ((lda % 2) != 0 || (ldb % 2) != 0)) return THL_ERR_INVALID;
  if (mx_out == MX_E2M1 && ldd % 2 != 0) return THL_ERR_INVALID;
  const bool work = m > 0 && n > 0 && bt.count > 0;
  if (work && mx_out != MX_NONE && (!sfd || ld_sfd < (m + 31) / 32)) return THL_ERR_INVALID;
  // Batched: the D matrices may not overlap one another; fp4 operands move
  // by whole bytes.
  if (work && bt.count > 1 && bt.d < (n - 1) * ldd + m) return THL_ERR_INVALID;
  if (fam == FAM_FP4 && (bt.a % 2 != 0 || bt.b % 2 != 0)) return THL_ERR_INVALID;
  if (work && !D) return THL_ERR_INVALID;
  if (work && k > 0 && (!A || !B)) return THL_ERR_INVALID;
  if (work && beta != 0.0f && !C) return THL_ERR_INVALID;
  if (work && has_bias && !bias) return THL_ERR_INVALID;
  const thl_scales unit_scales = {1.0f, 1.0f, nullptr, 0, nullptr, 0};
  const thl_scales& s = sc ? *sc : unit_scales;
  if (block_scaled && work && k > 0) {
    if (!s.sfa || !s.sfb) return THL_ERR_INVALID;
    if (s.ld_sfa < k / 32 || s.ld_sfb < k / 32) return THL_ERR_INVALID;
  }

  // ---- overlap: D may alias C exactly; nothing else may overlap D
  // (Batched: each array's whole span over the batch; a D that only
  // interleaves with another array is refused too.)
  if (work) {
    const int64_t L = bt.count;
    const Range rd = batch_range(D, dt->d, m, n, ldd, L, bt.d);
    if (overlaps(rd, batch_range(A, dt->a, rows_a, cols_a, lda, L, bt.a))) return THL_ERR_INVALID;
    if (overlaps(rd, batch_range(B, dt->b, rows_b, cols_b, ldb, L, bt.b))) return THL_ERR_INVALID;
    if (beta != 0.0f) {
      const bool exact_alias = (C == D) && (ldc == ldd) && (dt->c == dt->d) && (L == 1 || bt.c == bt.d);
      if (!exact_alias && overlaps(rd, batch_range(C, dt->c, m, n, ldc, L, bt.c))) return THL_ERR_INVALID;
    }
    if (has_bias && overlaps(rd, batch_range(bias, dt->bias, m, 1, m, L, bt.bias))) return THL_ERR_INVALID;
    if (block_scaled && k > 0) {
      if (overlaps(rd, batch_range(s.sfa, THL_E8M0, k / 32, m, s.ld_sfa, L, bt.sfa))) return THL_ERR_INVALID;
      if (overlaps(rd, batch_range(s.sfb, THL_E8M0, k / 32, n, s.ld_sfb, L, bt.sfb))) return THL_ERR_INVALID;
    }
    if (mx_out != MX_NONE) {
      // the generated scales overlap nothing else either
      const Range rs = matrix_range(sfd, THL_E8M0, (m + 31) / 32, n, ld_sfd);
      const Range others[] = {rd,
                              matrix_range(A, dt->a, rows_a, cols_a, lda),
                              matrix_range(B, dt->b, rows_b, cols_b, ldb),
                              beta != 0.0f ? matrix_range(C, dt->c, m, n, ldc) : Range{},
                              has_bias ? matrix_range(bias, dt->bias, m, 1, m) : Range{},
                              block_scaled && k > 0 ? matrix_range(s.sfa, THL_E8M0, k / 32, m, s.ld_sfa) : Range{},
                              block_scaled && k > 0 ? matrix_range(s.sfb, THL_E8M0, k / 32, n, s.ld_sfb) : Range{}};
      for (const Range& o : others)
        if (overlaps(rs, o)) return THL_ERR_INVALID;
    }
  }

  // Copy offsets inside a 256-row tile, and scale-row offsets, are 32-bit.
  if (k > 0 && (bytes_of(dt->a, lda) > (INT64_C(1) << 23) || bytes_of(dt->b, ldb) > (INT64_C(1) << 23)))
    return THL_ERR_UNSUPPORTED;
  if (block_scaled && k > 0 && (m * s.ld_sfa > (INT64_C(1) << 31) || n * s.ld_sfb > (INT64_C(1) << 31)))
    return THL_ERR_UNSUPPORTED;

  Prep& o = *out;
  o.fam = fam;
  o.a_kmajor = a_kmajor;
  o.b_kmajor = b_kmajor;
  o.block_scaled = block_scaled;
  o.int_path = int_path;
  o.has_bias = has_bias;
  o.small_m = m <= 64 && k > 0 && mx_out == MX_NONE;  // MX output: the tiled kernels' epilogue
  o.mx_out = mx_out;
  o.work = work;
  o.flags = flags;
  o.lda_bytes = bytes_of(dt->a, lda);
  o.ldb_bytes = bytes_of(dt->b, ldb);
  // Batched: every problem's base keeps the alignment of the first.
  o.sa_bytes = bt.count > 1 ? bytes_of(dt->a, bt.a) : 0;
  o.sb_bytes = bt.count > 1 ? bytes_of(dt->b, bt.b) : 0;
  o.s = s;
  // Vector epilogue: D, C and bias at their elements' alignment (a run of 8
  // elements moves as 16-byte accesses at any element offset, the memory
  // system being in unaligned mode), C 16-bit, and a 256-column panel within
  // 32-bit offsets.  rows16: every column run also a whole 16-byte unit.
  o.vec = false;
  if (!int_path && mx_out == MX_NONE) {
    auto unit16 = [](const void* ptr, int64_t ld_bytes) {
      return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0 && ld_bytes % 16 == 0 && ld_bytes <= (INT64_C(1) << 23);
    };
    auto elem_ok = [](const void* ptr, int64_t ld_bytes, int64_t e) {
      return reinterpret_cast<uintptr_t>(ptr) % e == 0 && ld_bytes % e == 0 && ld_bytes <= (INT64_C(1) << 23);
    };
    const int64_t ed = bytes_of(dt->d, 1), ec = beta != 0.0f ? bytes_of(dt->c, 1) : 1;
    const int64_t eb = has_bias ? bytes_of(dt->bias, 1) : 1;
    bool r16 = unit16(D, bytes_of(dt->d, ldd)), vec = elem_ok(D, bytes_of(dt->d, ldd), ed);
    if (beta != 0.0f) {
      r16 = r16 && unit16(C, bytes_of(dt->c, ldc));
      vec = vec && elem_ok(C, bytes_of(dt->c, ldc), ec) && (dt->c == THL_F16 || dt->c == THL_BF16);
    }
    if (has_bias) {
      r16 = r16 && (reinterpret_cast<uintptr_t>(bias) & 15) == 0;
      vec = vec && reinterpret_cast<uintptr_t>(bias) % eb == 0;
    }
    o.rows16 = r16;
    if (bt.count > 1) {
      const int64_t bs_c = beta != 0.0f ? bytes_of(dt->c, bt.c) : 0, bs_d = bytes_of(dt->d, bt.d);
      const int64_t bs_bias = has_bias ? bytes_of(dt->bias, bt.bias) : 0;
      if ((bs_c % ec) || (bs_d % ed) || (bs_bias % eb)) vec = false;
    }
    o.vec = vec;
  }
  return THL_OK;
}

// Does variant v take this problem's operands (alignment class, scale rows)?
bool fits(const Variant& v, const Prep& pr, const Batch& bt, const void* A, const void* B, int64_t k) {
  bool ok = k == 0 || (aligned(A, pr.lda_bytes, v.loadw) && aligned(B, pr.ldb_bytes, v.loadw) &&
                       pr.sa_bytes % v.loadw == 0 && pr.sb_bytes % v.loadw == 0);
  if (pr.block_scaled && k > 0)
    ok = ok && aligned(pr.s.sfa, pr.s.ld_sfa, 16) && aligned(pr.s.sfb, pr.s.ld_sfb, 16) &&
         (bt.count == 1 || (bt.sfa % 16 == 0 && bt.sfb % 16 == 0));
  return ok;
}

// The tile tier the shape rule prefers for this many tiles of each size:
// 256x256 from a whole round of them (one per CU); below that 128x128 while
// its tiles fit one round at two workgroups per CU, else 256x256 again, whose
// one partial round beats two of 128x128.  Measured on one box (bf16 N/N
// relu(A B + C + bias); e4m3 T/N): 3072^3, 144 tiles of 256x256 and 576 of
// 128x128: 62.7 us on 256x256 against 77.8 on 128x128 and 81.5 on 256x128;
// e4m3 36.4, 43.8 and 49.9 us.  3584^3: 81.0, 94.1 and 99.7 us; e4m3 43.4,
// 51.4 and 59.4 us.
// A float problem that reads C through the general epilogue (an fp32 C,
// which the vector epilogue does not read) with D, C or bias column runs off
// 16-byte units (an odd leading dimension, say) takes it on every tile, its
// C loads waiting block by block; with one workgroup per CU nothing hides
// them, so it starts at the two-workgroup tiers.  Measured with ldd = ldc =
// 4097, bf16 4096^3 relu(A B + C + bias) with fp32 C: 134.2 us on 256x128
// against 144.2 on 256x256.
int want_tier_of(int64_t tiles_256, int64_t tiles_128, bool general_epilogue = false) {
  int64_t ncu = cu_count();
  if (ncu <= 0) ncu = 256;
  const int t = tiles_256 >= ncu ? 0 : (tiles_128 <= 2 * ncu ? 2 : 0);
  return general_epilogue && t == 0 ? 1 : t;
}

// First fit over the built variants of the problem's family, in the order
// of the shape rule: the small-M kernel where it applies (allow_small),
// then the preferred tier, then each smaller tile, then any tiled variant;
// `fit` decides alignment.  The one-workgroup 128x128 variants only where
// `one_round` says the launch's 128x128 tiles all run at once, one per CU:
// then no second workgroup is there to hide a tile's load latency, and their
// deeper ring (six stages instead of four) does instead.  Measured (bf16 N/N
// relu(A B + C + bias), steady clock, three rounds in fresh processes):
// 2048^3 28.2 -> 23.6 us, 1536^3 20.7 -> 19.0, 4096 x 1024 x 4096 46.8 ->
// 40.1; e4m3 T/N 2048^3 13.1 -> 12.1; int8 equal.  With more tiles than CUs
// the two-workgroup variants win (2560^3, 400 tiles: 39 against 53 us).
// THL_FORCE_VARIANT=<name> restricts the choice to that variant.  Returns
// nullptr with *status set when none fits.
template <class Fit>
const Variant* choose_variant(const Prep& pr, bool allow_small, int64_t rows, int want_tier, bool one_round,
                              Fit&& fit, thl_status* status) {
  const char* forced = std::getenv("THL_FORCE_VARIANT");
  const bool small_m = allow_small && pr.small_m;
  const Variant* pick = nullptr;
  bool family_built = false;
  for (int pass = small_m ? -1 : want_tier; pass <= 3 && !pick; pass = pass < 0 ? want_tier : pass + 1) {
    for (const Variant& v : kVariants) {
      if (v.family != pr.fam || v.a_kmajor != pr.a_kmajor || v.b_kmajor != pr.b_kmajor) continue;
      family_built = true;
      if (forced && *forced) {
        if (std::strcmp(forced, v.name) != 0 || (v.tier < 0 && (!small_m || v.bm < rows))) continue;
      } else if ((pass < 3 && v.tier != pass) || (pass == 3 && v.tier < 0) || (v.tier < 0 && v.bm < rows) ||
                 (v.tier == 2 && v.occ == 1 && !one_round)) {
        continue;
      }
      // MX-format D runs on the MX-output variants, and only it does
      if ((pr.mx_out != MX_NONE) != v.mxout) continue;
      if (fit(v)) {
        pick = &v;
        break;
      }
    }
    if (forced && *forced) break;
  }
  if (!pick) *status = (forced && *forced) ? THL_ERR_UNSUPPORTED : (family_built ? THL_ERR_MISALIGNED : THL_ERR_UNSUPPORTED);
  return pick;
}

// Kernel arguments of one problem for variant v.
GemmArgs make_args(const Prep& pr, const Variant& v, int64_t m, int64_t n, int64_t k, const void* A, const void* B,
                   const void* C, int64_t ldc, void* D, int64_t ldd, float alpha, float beta, const thl_dtypes* dt,
                   const void* bias) {
  GemmArgs a{};
  a.a = static_cast<const uint8_t*>(A);
  a.b = static_cast<const uint8_t*>(B);
  a.c = C;
  a.d = D;
  a.bias = pr.has_bias ? bias : nullptr;
  a.sfa = pr.s.sfa;
  a.sfb = pr.s.sfb;
  a.lda_bytes = pr.lda_bytes;
  a.ldb_bytes = pr.ldb_bytes;
  a.ldc = ldc;
  a.ldd = ldd;
  a.ld_sfa = pr.s.ld_sfa;
  a.ld_sfb = pr.s.ld_sfb;
  a.m = static_cast<int32_t>(m);
  a.n = static_cast<int32_t>(n);
  a.k = static_cast<int32_t>(k);
  a.kbytes = static_cast<int32_t>(bytes_of(dt->a, k));
  a.tiles_m = static_cast<int32_t>((m + v.bm - 1) / v.bm);
  a.tiles_n = static_cast<int32_t>((n + v.bn - 1) / v.bn);
  a.group_m = 8;
  const bool tensor_scaled = (dt->a == THL_E4M3 || dt->a == THL_E5M2) && (dt->b == THL_E4M3 || dt->b == THL_E5M2);
  a.alpha = tensor_scaled ? alpha * pr.s.a_scale * pr.s.b_scale : alpha;
  a.beta = beta;
  a.flags = static_cast<int32_t>(pr.flags) | (pr.vec ? EPI_VEC : 0);
  a.c_type = static_cast<int32_t>(dt->c);
  a.d_type = static_cast<int32_t>(dt->d);
  a.bias_type = static_cast<int32_t>(dt->bias);
  a.mx_out = pr.mx_out;
  return a;
}

// Persistent workgroups for `problems` grid rows: at most as many as the
// device holds at once, shared out over the rows (a multiple of 8 per row
// while that many fit, so each XCD keeps its own range of tiles), and no
// more than the largest row's tile count.  0 when the device cannot be
// queried.
int64_t persistent_grid(const Variant& v, int64_t problems, int64_t max_tiles) {
  const int ncu = cu_count();
  if (ncu <= 0) return 0;
  const int64_t resident = static_cast<int64_t>(ncu) * v.occ;
  int64_t per = resident / problems;
  if (per >= 8) per -= per % 8;
  if (per < 1) per = 1;
  return max_tiles < per ? max_tiles : per;
}

// Splits for one problem on variant v: only the variants built with split K
// (128x128, two workgroups per CU, unscaled families) and a single problem.
// Splitting pays when the tiles fill at most an eighth of the resident
// workgroups and K is long (at least 128 K-steps): then as many splits as
// fill them, at most 16, with at least 16 K-steps each.  Measured on bf16
// and fp8 with K = 8192: 64 tiles went from 79 to 41 us (bf16) and 44 to
// 32 us (fp8), 15 tiles from 81 to 30 us (fp16); at 256 tiles, or K of 64
// steps, the partial matrices' traffic and the second kernel cost more than
// the split gains.  At 128 tiles (256 x 8192 x 8192) the unsplit six-stage
// variant is faster than 4 splits: bf16 58.2 against 64.3 us, e4m3 34.0
// against 42.6; at 64 tiles 8 splits still beat it for bf16 (42.6 against
// 55.9 us) and tie for e4m3 (32.4 against 33.1).  THL_FORCE_SPLITS=<s> asks for s splits on any eligible
// variant (tests use it to cover the path at small sizes).
int splits_for(const Prep& pr, const Batch& bt, int64_t tiles, int64_t kbytes);

int choose_splits(const Prep& pr, const Variant& v, const Batch& bt, int64_t tiles, int64_t kbytes) {
  if (v.tier < 0 || v.occ != 2 || v.bm * v.bn > 128 * 128) return 1;
  return splits_for(pr, bt, tiles, kbytes);
}

// The splits choose_splits gives a split-K variant for `tiles` tiles.
int splits_for(const Prep& pr, const Batch& bt, int64_t tiles, int64_t kbytes) {
  if (bt.count != 1 || pr.block_scaled || kbytes <= 0 || pr.mx_out != MX_NONE) return 1;
  const int64_t nk_all = (kbytes + 63) / 64;
  const char* forced = std::getenv("THL_FORCE_SPLITS");
  if (forced && *forced) {
    const int64_t f = std::atoll(forced);
    return static_cast<int>(f < 1 ? 1 : (f > nk_all ? nk_all : (f > 64 ? 64 : f)));
  }
  const int ncu = cu_count();
  const int64_t resident = static_cast<int64_t>(ncu) * 2;
  if (ncu <= 0 || tiles * 8 > resident || nk_all < 128) return 1;
  int64_t sp = resident / tiles;
  if (sp > nk_all / 16) sp = nk_all / 16;
  if (sp > 16) sp = 16;
  return sp >= 2 ? static_cast<int>(sp) : 1;
}

// Operands the tiled kernels cannot stage directly are first rewritten as
// K-major rows (convert.hip): 8-bit operands stored along M (N), 6-bit
// operands, 4-bit operands beside another format or without block scales.
// Stage says which operand is rewritten and into which format.
struct Stage {
  bool a = false, b = false;
  thl_dtype ta = THL_NONE, tb = THL_NONE;  // formats after the rewrite
  // 16-bit operands: lines re-pitched byte for byte in their own layout
  // (M- or K-major kept) rather than rewritten as K-major rows
  bool keep_a = false, keep_b = false;
};

bool is_fp8(thl_dtype t) { return t == THL_E4M3 || t == THL_E5M2; }
bool is_narrow_float(thl_dtype t) { return is_fp8(t) || t == THL_E2M1X2 || t == THL_E2M3 || t == THL_E3M2; }

// True when the problem takes the conversion pass (and fills *sg); false
// for every combination the kernels stage directly and for the ones no path
// builds (validation then reports those).  A K-major 8- or 4-bit operand
// whose rows are not 16-byte aligned is rewritten too (into 64-byte rows)
// when D has 2^23 elements or more: only the 4-byte-copy kernels could
// stage it as it is, and with many tiles they run at half the 16-byte
// kernels' rate.  Measured on fp8 rows 8 bytes past a 16-byte unit: 8192^3
// 1007 us on the 4-byte kernel against 488 us rewritten, 4096^3 144 against
// 96 us; with few tiles the 16-byte kernel is bound by load latency as well
// and the pass does not pay (4097 x 1000 x 2040: 44.6 against 57.1 us, and
// since the epilogue's element-aligned accesses 34.4 us on the 4-byte
// kernel; 2048 x 2048 x 8192: 76 against 83 us).
bool plan_stage(const thl_dtypes* dt, thl_op opA, thl_op opB, const thl_scales* sc, int64_t m, int64_t n, int64_t k,
                const void* A, int64_t lda, const void* B, int64_t ldb, const Batch& bt, Stage* sg) {
  if (!dt) return false;
  const bool a_km = opA == THL_OP_T, b_km = opB == THL_OP_N;
  Stage g;
  if (dt->a == THL_I8 && dt->b == THL_I8) {
    g.a = !a_km;
    g.b = !b_km;
    g.ta = g.tb = THL_I8;
  } else if (is_narrow_float(dt->a) && is_narrow_float(dt->b)) {
    const bool any_sf = sc && (sc->sfa || sc->sfb);
    if (dt->a == THL_E2M1X2 && dt->b == THL_E2M1X2 && any_sf) {
      // MXFP4 both sides: fp4 rows (nibbles moved, not widened)
      g.a = !a_km;
      g.b = !b_km;
      g.ta = g.tb = THL_E2M1X2;
    } else {
      // fp8 rows for the fp8 kernels: fp8 stays itself, the others widen to E4M3
      g.a = !(is_fp8(dt->a) && a_km);
      g.b = !(is_fp8(dt->b) && b_km);
      g.ta = is_fp8(dt->a) ? dt->a : THL_E4M3;
      g.tb = is_fp8(dt->b) ? dt->b : THL_E4M3;
    }
  } else if (!((dt->a == THL_F16 || dt->a == THL_BF16) && dt->b == dt->a)) {
    return false;
  }
  // re-pitch misaligned K-major rows of a large problem (not when a variant
  // is forced: THL_FORCE_VARIANT keeps the caller's operands as they are)
  const char* forced = std::getenv("THL_FORCE_VARIANT");
  const bool large = k > 0 && m * n >= (INT64_C(1) << 23) && !(forced && *forced);
  auto rows16 = [&](const void* p, thl_dtype t, int64_t ld, int64_t stride) {
    return reinterpret_cast<uintptr_t>(p) % 16 == 0 && bytes_of(t, ld) % 16 == 0 &&
           (bt.count <= 1 || bytes_of(t, stride) % 16 == 0);
  };
  // rows that are not even whole 4-byte units fit no kernel at all: rewritten
  // whatever the size
  auto rows4 = [&](const void* p, thl_dtype t, int64_t ld, int64_t stride) {
    return reinterpret_cast<uintptr_t>(p) % 4 == 0 && bytes_of(t, ld) % 4 == 0 &&
           (bt.count <= 1 || bytes_of(t, stride) % 4 == 0);
  };
  auto repitchable = [](thl_dtype t) { return t == THL_I8 || is_fp8(t) || t == THL_E2M1X2; };
  const bool keep = forced && *forced;
  // lines no kernel reads: not whole 4-byte units, or for MX-format D (whose
  // kernels load 16-byte units only) not whole 16-byte units
  const bool mx_d = is_mx_out(dt->d);
  auto unreadable = [&](const void* p, thl_dtype t, int64_t ld, int64_t stride) {
    return mx_d ? !rows16(p, t, ld, stride) : !rows4(p, t, ld, stride);
  };
  if (dt->a == THL_F16 || dt->a == THL_BF16) {
    // 16-bit lines (rows along K, or k-lines along M) in either layout, by
    // the same rules: lines no kernel reads, or not whole 16-byte units with
    // D of 2^23 elements or more
    g.a = (large && !rows16(A, dt->a, lda, bt.a)) || (!keep && unreadable(A, dt->a, lda, bt.a));
    g.b = (large && !rows16(B, dt->b, ldb, bt.b)) || (!keep && unreadable(B, dt->b, ldb, bt.b));
    g.ta = dt->a;
    g.tb = dt->b;
    g.keep_a = g.a;
    g.keep_b = g.b;
    if (!g.a && !g.b) return false;
    *sg = g;
    return true;
  }
  if (!g.a && a_km && repitchable(dt->a) &&
      ((large && !rows16(A, dt->a, lda, bt.a)) || (!keep && unreadable(A, dt->a, lda, bt.a)))) {
    g.a = true;
    g.ta = dt->a;
  }
  if (!g.b && b_km && repitchable(dt->b) &&
      ((large && !rows16(B, dt->b, ldb, bt.b)) || (!keep && unreadable(B, dt->b, ldb, bt.b)))) {
    g.b = true;
    g.tb = dt->b;
  }
  if (!g.a && !g.b) return false;
  *sg = g;
  return true;
}

thl_status static_scratch(hipStream_t stream, int64_t bytes, uint8_t** out);
thl_status staged_gemm(const Batch& bt, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda,
                       thl_op opA, const void* B, int64_t ldb, thl_op opB, const void* C, int64_t ldc, void* D,
                       int64_t ldd, float alpha, float beta, const thl_dtypes* dt, const thl_epilogue* epi,
                       const thl_scales* sc, struct ihipStream_t* stream, int ws_mode, int64_t ws_offset,
                       const struct Stage& sg);

thl_status gemm_impl(const Batch& bt, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda, thl_op opA,
                     const void* B, int64_t ldb, thl_op opB, const void* C, int64_t ldc, void* D, int64_t ldd,
                     float alpha, float beta, const thl_dtypes* dt, const thl_epilogue* epi, const thl_scales* sc,
                     struct ihipStream_t* stream, int ws_mode, int64_t ws_offset) {
  Stage sg;
  if (plan_stage(dt, opA, opB, sc, m, n, k, A, lda, B, ldb, bt, &sg))
    return staged_gemm(bt, m, n, k, A, lda, opA, B, ldb, opB, C, ldc, D, ldd, alpha, beta, dt, epi, sc, stream, ws_mode,
                       ws_offset, sg);
  Prep pr;
  const unsigned flags = epi ? epi->flags : 0u;
  thl_status st = prepare(bt, m, n, k, A, lda, opA, B, ldb, opB, C, ldc, D, ldd, alpha, beta, dt, flags,
                          epi ? epi->bias : nullptr, sc, epi ? epi->sfd : nullptr, epi ? epi->ld_sfd : 0, &pr);
  if (st != THL_OK) return st;

  // ---- variant: first fit on family, alignment and shape
  // (tile counts over the whole batch: its problems fill the device together)
  const int64_t tiles_256 = ((m + 255) / 256) * ((n + 255) / 256) * bt.count;
  const int64_t tiles_128 = ((m + 127) / 128) * ((n + 127) / 128) * bt.count;
  const int want =
      want_tier_of(tiles_256, tiles_128, !pr.int_path && !pr.vec && !pr.rows16 && pr.mx_out == MX_NONE && beta != 0.0f);

  // ---- a last round of 256x256 tiles that would leave most CUs idle: the
  // rows of whole rounds run first, the remaining rows as a problem of their
  // own (smaller tiles, the whole chip).  6144^3 makes 576 tiles, 2.25 rounds
  // of 256 CUs: run as 504 tiles, then 768 rows on 128x128 tiles.
  if (want == 0 && bt.count == 1 && pr.work && !pr.small_m && pr.mx_out == MX_NONE) {
    const char* forced = std::getenv("THL_FORCE_VARIANT");
    const int64_t ncu = cu_count();
    const int64_t tn = (n + 255) / 256;
    if (!(forced && *forced) && ncu > 0 && tiles_256 >= ncu && (tiles_256 % ncu) * 2 <= ncu &&
        tiles_256 % ncu != 0) {
      const int64_t rows = (tiles_256 / ncu) * ncu / tn * 256;  // whole tile rows within the full rounds
      if (rows > 0 && rows < m) {
        const int64_t off_a = opA == THL_OP_N ? bytes_of(dt->a, rows) : bytes_of(dt->a, rows * lda);
        const uint8_t* a_rest = static_cast<const uint8_t*>(A) + off_a;
        const uint8_t* c_rest = C ? static_cast<const uint8_t*>(C) + bytes_of(dt->c, rows) : nullptr;
        uint8_t* d_rest = static_cast<uint8_t*>(D) + bytes_of(dt->d, rows);
        thl_epilogue e2 = epi ? *epi : thl_epilogue{0u, nullptr, nullptr, 0};
        if (e2.bias) e2.bias = static_cast<const uint8_t*>(e2.bias) + bytes_of(dt->bias, rows);
        thl_scales s2 = sc ? *sc : thl_scales{1.0f, 1.0f, nullptr, 0, nullptr, 0};
        if (s2.sfa) s2.sfa += rows * s2.ld_sfa;
        st = gemm_impl(bt, rows, n, k, A, lda, opA, B, ldb, opB, C, ldc, D, ldd, alpha, beta, dt, epi, sc, stream,
                       ws_mode, ws_offset);
        if (st != THL_OK) return st;
        char first[128];
        std::snprintf(first, sizeof(first), "%s", t_last_variant);
        st = gemm_impl(bt, m - rows, n, k, a_rest, lda, opA, B, ldb, opB, c_rest, ldc, d_rest, ldd, alpha, beta, dt,
                       epi ? &e2 : nullptr, sc ? &s2 : nullptr, stream, ws_mode, ws_offset);
        if (st != THL_OK) return st;
        std::snprintf(t_rows_name, sizeof(t_rows_name), "%s|%s", first, t_last_variant);
        t_last_variant = t_rows_name;
        return THL_OK;
      }
    }
  }
  const int ncu = cu_count();
  const int64_t kbytes = bytes_of(dt->a, k);
  const int splits_128 = splits_for(pr, bt, tiles_128, kbytes);
  const bool one_round = want == 2 && ncu > 0 && tiles_128 <= ncu && splits_128 == 1;
  // The small-M kernel re-reads all of A from L2 in every 16-column
  // workgroup, a cost that grows with M x N x K; split K over 128x128 tiles
  // costs about the same at any M up to 128.  From M x N x K bytes of 3 GiB,
  // where K splits, the tiles win.  Measured at N = K = 8192 (small-M kernel
  // against 128x128 tiles with 8 splits): bf16 M = 24 42.5 against 36.0 us,
  // M = 32 48.1 against 36.7, M = 64 80.1 against 43.7; e4m3 M = 48 34.3
  // against 32.5, M = 64 39.9 against 33.4; int8 M = 64 39.3 against 26.6.
  // Below it the small-M kernel wins: e4m3 M = 33 28.9 against 32.4, and at
  // N = K = 4096 every M up to 64 (bf16 M = 64 26.2 against 29.6 us).
  const bool small_m_kernel = !(pr.small_m && splits_128 > 1 && m * n * kbytes >= (INT64_C(3) << 30));
  const Variant* pick = choose_variant(pr, small_m_kernel, m, want, one_round,
                                       [&](const Variant& v) { return fits(v, pr, bt, A, B, k); }, &st);
  if (!pick) return st;
  if (!pr.work) {
    t_last_variant = pick->name;
    last_splits = 1;
    return THL_OK;
  }

  // ---- launch
  GemmArgs a = make_args(pr, *pick, m, n, k, A, B, C, ldc, D, ldd, alpha, beta, dt, epi ? epi->bias : nullptr);
  if (pr.mx_out != MX_NONE) {
    a.sfd = epi->sfd;
    a.ld_sfd = epi->ld_sfd;
  }
  // Batch strides in bytes (zero for a single problem and for absent arrays).
  if (bt.count > 1) {
    a.bs_a = pr.sa_bytes;
    a.bs_b = pr.sb_bytes;
    a.bs_c = beta != 0.0f ? bytes_of(dt->c, bt.c) : 0;
    a.bs_d = bytes_of(dt->d, bt.d);
    a.bs_bias = pr.has_bias ? bytes_of(dt->bias, bt.bias) : 0;
    a.bs_sfa = pr.block_scaled ? bt.sfa : 0;
    a.bs_sfb = pr.block_scaled ? bt.sfb : 0;
  }
  if (pick->tier < 0) {  // small M: one workgroup per 16 columns
    if (pick->launch(a, dim3(static_cast<unsigned>((n + 15) / 16), static_cast<unsigned>(bt.count)),
                     reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
      return THL_ERR_HIP;
    t_last_variant = pick->name;
    last_splits = 1;
    return THL_OK;
  }
  const int64_t tiles = static_cast<int64_t>(a.tiles_m) * a.tiles_n;
  if (tiles > INT32_MAX) return THL_ERR_UNSUPPORTED;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  // Split K over workgroups when the tiles fill at most half the resident
  // workgroups: each tile's K-steps go to `splits` consecutive units.
  int splits = choose_splits(pr, *pick, bt, tiles, a.kbytes);
  uint8_t* ws = nullptr;
  bool pooled = false;
  const int64_t ld_ws = (m + 3) / 4 * 4;                      // 16-byte columns
  const int64_t stride = (ld_ws * n * 4 + 255) / 256 * 256;  // bytes per split
  if (splits > 1) {
    const int64_t nk_all = (a.kbytes + 63) / 64;
    const int64_t ksteps = (nk_all + splits - 1) / splits;
    splits = static_cast<int>((nk_all + ksteps - 1) / ksteps);  // no empty split
    a.ksteps = static_cast<int32_t>(ksteps);
    const int64_t bytes = splits * stride;
    if (ws_mode == WS_STATIC) {
      st = static_scratch(hs, ws_offset + bytes, &ws);
      if (st != THL_OK) return st;
      ws += ws_offset;  // past what the caller holds
    } else {
      int dev = 0;
      hipMemPool_t pool = hipGetDevice(&dev) == hipSuccess ? pool_for_device(dev) : nullptr;
      if (pool && hipMallocFromPoolAsync(reinterpret_cast<void**>(&ws), static_cast<size_t>(bytes), pool, hs) ==
                      hipSuccess) {
        pooled = true;
      } else {
        (void)hipGetLastError();
        ws = nullptr;  // no workspace: run unsplit
      }
    }
    if (!ws) splits = 1;
  }
  const int64_t units = tiles * splits;
  // Persistent workgroups; each walks units blockIdx.y, + gridDim.y, ...
  const int64_t grid = persistent_grid(*pick, bt.count, units);
  if (grid <= 0) {
    if (pooled) (void)hipFreeAsync(ws, hs);
    return THL_ERR_HIP;
  }
  hipError_t le;
  if (splits > 1) {
    // the splits' partial products, unscaled, to the workspace ...
    GemmArgs ap = a;
    ap.splits = splits;
    ap.split_stride = stride;
    ap.d = ws;
    ap.ldd = ld_ws;
    ap.d_type = pr.int_path ? THL_I32 : THL_F32;
    ap.c = nullptr;
    ap.bias = nullptr;
    ap.alpha = 1.0f;
    ap.beta = 0.0f;
    ap.flags = pr.int_path ? 0 : EPI_VEC;
    le = pick->launch(ap, dim3(1u, static_cast<unsigned>(grid)), hs);
    // ... then their sum in split order through the epilogue
    if (le == hipSuccess) {
      ReduceArgs r{};
      r.ws = ws;
      r.ld_ws = ld_ws;
      r.stride = stride;
      r.splits = splits;
      r.m = a.m;
      r.n = a.n;
      r.int_path = pr.int_path ? 1 : 0;
      r.c = a.c;
      r.ldc = a.ldc;
      r.c_type = a.c_type;
      r.bias = a.bias;
      r.bias_type = a.bias_type;
      r.d = a.d;
      r.ldd = a.ldd;
      r.d_type = a.d_type;
      r.alpha = a.alpha;
      r.beta = a.beta;
      r.flags = static_cast<int32_t>(pr.flags);
      const int64_t chunks = (m + 3) / 4 * n;
      const int64_t blocks = (chunks + 255) / 256 < 4096 ? (chunks + 255) / 256 : 4096;
      hipLaunchKernelGGL(splitk_reduce, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, hs, r);
      le = hipGetLastError();
    }
  } else {
    a.xcd_local = bt.count % 8 == 0 ? 1 : 0;
    le = pick->launch(a, dim3(static_cast<unsigned>(bt.count), static_cast<unsigned>(grid)), hs);
  }
  if (pooled) (void)hipFreeAsync(ws, hs);  // back to the pool once the kernels have run
  if (le != hipSuccess) return THL_ERR_HIP;
  t_last_variant = pick->name;
  last_splits = splits;
  return THL_OK;
}

// Bytes of one rewritten operand row: whole 64-byte K-steps of the target format.
int64_t staged_ld_bytes(thl_dtype t, int64_t k) {
  const int64_t b = bytes_of(t, k);
  return b <= 0 ? 64 : (b + 63) / 64 * 64;
}

thread_local char t_staged_name[192];

// The problem with the operands in sg rewritten (convert.hip) into a
// workspace and then run as a K-major problem of the rewritten formats.  The
// caller's operands are validated here (what the K-major run cannot see:
// their shapes, leading dimensions, pointers and overlap with D); everything
// else is validated by the K-major run.  Per-tensor scales stay with fp8
// operands; E2M1, E2M3 and E3M2 operands take none (as 1).
thl_status staged_gemm(const Batch& bt, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda, thl_op opA,
                       const void* B, int64_t ldb, thl_op opB, const void* C, int64_t ldc, void* D, int64_t ldd,
                       float alpha, float beta, const thl_dtypes* dt, const thl_epilogue* epi, const thl_scales* sc,
                       struct ihipStream_t* stream, int ws_mode, int64_t ws_offset, const Stage& sg) {
  if (m < 0 || n < 0 || k < 0 || bt.count < 0 || bt.a < 0 || bt.b < 0) return THL_ERR_INVALID;
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX || lda > INT32_MAX || ldb > INT32_MAX) return THL_ERR_UNSUPPORTED;
  if (bt.count > 65535 || bt.a > (INT64_C(1) << 40) || bt.b > (INT64_C(1) << 40)) return THL_ERR_UNSUPPORTED;
  const int64_t rows_a = (opA == THL_OP_N) ? m : k, cols_a = (opA == THL_OP_N) ? k : m;
  const int64_t rows_b = (opB == THL_OP_N) ? k : n, cols_b = (opB == THL_OP_N) ? n : k;
  if (lda < (rows_a > 1 ? rows_a : 1) || ldb < (rows_b > 1 ? rows_b : 1)) return THL_ERR_INVALID;
  // a stored line (and each problem of a batch) starts on a whole byte
  auto whole_bytes = [](thl_dtype t, int64_t elems) { return (elems * bits_of(t)) % 8 == 0; };
  if (!whole_bytes(dt->a, lda) || !whole_bytes(dt->b, ldb) || !whole_bytes(dt->a, bt.a) || !whole_bytes(dt->b, bt.b))
    return THL_ERR_INVALID;
  const bool work = m > 0 && n > 0 && bt.count > 0;
  if (work && k > 0 && (!A || !B)) return THL_ERR_INVALID;
  if (work && D) {
    const Range rd = batch_range(D, dt->d, m, n, ldd, bt.count, bt.d);
    if (overlaps(rd, batch_range(A, dt->a, rows_a, cols_a, lda, bt.count, bt.a)) ||
        overlaps(rd, batch_range(B, dt->b, rows_b, cols_b, ldb, bt.count, bt.b)))
      return THL_ERR_INVALID;
    if (epi && epi->sfd && is_mx_out(dt->d) && m > 0) {
      const Range rs = matrix_range(epi->sfd, THL_E8M0, (m + 31) / 32, n, epi->ld_sfd);
      if (overlaps(rs, matrix_range(A, dt->a, rows_a, cols_a, lda)) ||
          overlaps(rs, matrix_range(B, dt->b, rows_b, cols_b, ldb)))
        return THL_ERR_INVALID;
    }
  }
  // ---- the rewritten operands: K-major rows of 64-byte steps, or (16-bit,
  // keep_*) the caller's lines, in the caller's layout, at a pitch of whole
  // 64-byte units.  lines_* lines of line_*: A's are rows (opA = T) or
  // k-lines along M (opA = N), B's columns (opB = N) or k-lines along N.
  const int64_t lines_a = sg.keep_a && opA == THL_OP_N ? k : m;
  const int64_t lines_b = sg.keep_b && opB == THL_OP_T ? k : n;
  const int64_t line_a = sg.keep_a && opA == THL_OP_N ? m : k;
  const int64_t line_b = sg.keep_b && opB == THL_OP_T ? n : k;
  if (sg.a && (lines_a + 63) / 64 > 65535) return THL_ERR_UNSUPPORTED;  // the pass's grid
  if (sg.b && (lines_b + 63) / 64 > 65535) return THL_ERR_UNSUPPORTED;
  const int64_t lda_b = staged_ld_bytes(sg.ta, line_a), ldb_b = staged_ld_bytes(sg.tb, line_b);
  const int64_t elems_per_byte_a = sg.ta == THL_E2M1X2 ? 2 : 1, elems_per_byte_b = sg.tb == THL_E2M1X2 ? 2 : 1;
  const int64_t elem_bytes_a = sg.keep_a ? 2 : 1, elem_bytes_b = sg.keep_b ? 2 : 1;  // kept 16-bit elements
  const int64_t size_a = sg.a ? (lines_a * lda_b + 255) / 256 * 256 : 0;
  const int64_t size_b = sg.b ? (lines_b * ldb_b + 255) / 256 * 256 : 0;
  const int64_t count = bt.count > 0 ? bt.count : 0;
  const int64_t total = count * (size_a + size_b);
  const bool run_pass = work && k > 0 && total > 0;
  // ---- the K-major problem, validated before the pass runs
  thl_dtypes d2 = *dt;
  if (sg.a) d2.a = sg.ta;
  if (sg.b) d2.b = sg.tb;
  thl_scales s2 = sc ? *sc : thl_scales{1.0f, 1.0f, nullptr, 0, nullptr, 0};
  if (!is_fp8(dt->a)) s2.a_scale = 1.0f;
  if (!is_fp8(dt->b)) s2.b_scale = 1.0f;
  Batch b2 = bt;
  if (sg.a) b2.a = count > 1 ? size_a * elems_per_byte_a / elem_bytes_a : 0;
  if (sg.b) b2.b = count > 1 ? size_b * elems_per_byte_b / elem_bytes_b : 0;
  // The rewritten operands are fresh memory: validated at stand-in addresses
  // (256-byte aligned, far above any allocation, never dereferenced) so that
  // every argument error is reported before anything is allocated or run.
  const uintptr_t stand_in = static_cast<uintptr_t>(1) << 62;
  const void* A2 = sg.a ? (run_pass ? reinterpret_cast<const void*>(stand_in) : nullptr) : A;
  const void* B2 = sg.b ? (run_pass ? reinterpret_cast<const void*>(stand_in + count * size_a) : nullptr) : B;
  const int64_t lda2 = sg.a ? lda_b * elems_per_byte_a / elem_bytes_a : lda;
  const int64_t ldb2 = sg.b ? ldb_b * elems_per_byte_b / elem_bytes_b : ldb;
  const thl_op opA2 = sg.a && !sg.keep_a ? THL_OP_T : opA, opB2 = sg.b && !sg.keep_b ? THL_OP_N : opB;
  {
    Prep check;
    const thl_status st = prepare(b2, m, n, k, A2, lda2, opA2, B2, ldb2, opB2, C, ldc, D, ldd, alpha, beta, &d2,
                                  epi ? epi->flags : 0u, epi ? epi->bias : nullptr, sc ? &s2 : nullptr,
                                  epi ? epi->sfd : nullptr, epi ? epi->ld_sfd : 0, &check);
    if (st != THL_OK) return st;
  }

  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = nullptr;
  bool pooled = false;
  if (run_pass) {
    if (ws_mode == WS_STATIC) {
      const thl_status st = static_scratch(hs, ws_offset + total, &ws);
      if (st != THL_OK) return st;
      ws += ws_offset;
    } else {
      int dev = 0;
      hipMemPool_t pool = hipGetDevice(&dev) == hipSuccess ? pool_for_device(dev) : nullptr;
      if (!pool || hipMallocFromPoolAsync(reinterpret_cast<void**>(&ws), static_cast<size_t>(total), pool, hs) !=
                       hipSuccess) {
        (void)hipGetLastError();
        return THL_ERR_HIP;
      }
      pooled = true;
    }
  }
  uint8_t* wa = ws;
  uint8_t* wb = ws ? ws + count * size_a : nullptr;
  if (run_pass && sg.a) A2 = wa;
  if (run_pass && sg.b) B2 = wb;

  // ---- the pass
  auto pass = [&](const void* src, thl_dtype from, thl_dtype to, int64_t ld, int64_t stride, bool kmajor, int64_t rows,
                  uint8_t* dst, int64_t dst_ld, int64_t dst_batch) -> hipError_t {
    CvtArgs c{};
    c.src = static_cast<const uint8_t*>(src);
    c.ld_bytes = bytes_of(from, ld);
    c.line_bytes = bytes_of(from, kmajor ? k : rows);
    c.src_batch = bytes_of(from, stride);
    c.src_fmt = from;
    c.dst_fmt = to;
    c.kmajor = kmajor ? 1 : 0;
    c.aligned4 = (reinterpret_cast<uintptr_t>(src) % 4 == 0 && c.ld_bytes % 4 == 0 && c.src_batch % 4 == 0) ? 1 : 0;
    c.rows = rows;
    c.k = k;
    c.dst = dst;
    c.dst_ld_bytes = dst_ld;
    c.dst_batch = dst_batch;
    return launch_convert(c, count, hs);
  };
  // 16-bit lines moved byte for byte: the pass's 8-bit K-major path over
  // lines of 2 * line bytes
  auto repitch = [&](const void* src, int64_t ld, int64_t stride, int64_t lines, int64_t line, uint8_t* dst,
                     int64_t dst_ld, int64_t dst_batch) -> hipError_t {
    CvtArgs c{};
    c.src = static_cast<const uint8_t*>(src);
    c.ld_bytes = 2 * ld;
    c.line_bytes = 2 * line;
    c.src_batch = 2 * stride;
    c.src_fmt = THL_I8;
    c.dst_fmt = THL_I8;
    c.kmajor = 1;
    c.aligned4 = (reinterpret_cast<uintptr_t>(src) % 4 == 0 && c.ld_bytes % 4 == 0 && c.src_batch % 4 == 0) ? 1 : 0;
    c.rows = lines;
    c.k = 2 * line;
    c.dst = dst;
    c.dst_ld_bytes = dst_ld;
    c.dst_batch = dst_batch;
    return launch_convert(c, count, hs);
  };
  hipError_t le = hipSuccess;
  if (run_pass && sg.a)
    le = sg.keep_a ? repitch(A, lda, bt.a, lines_a, line_a, wa, lda_b, size_a)
                   : pass(A, dt->a, sg.ta, lda, bt.a, opA == THL_OP_T, m, wa, lda_b, size_a);
  if (run_pass && sg.b && le == hipSuccess)
    le = sg.keep_b ? repitch(B, ldb, bt.b, lines_b, line_b, wb, ldb_b, size_b)
                   : pass(B, dt->b, sg.tb, ldb, bt.b, opB == THL_OP_N, n, wb, ldb_b, size_b);
  if (le != hipSuccess) {
    if (pooled) (void)hipFreeAsync(ws, hs);
    return THL_ERR_HIP;
  }

  // ---- the K-major run
  const thl_status st = gemm_impl(b2, m, n, k, A2, lda2, opA2, B2, ldb2, opB2, C, ldc, D, ldd, alpha, beta, &d2, epi,
                                  sc ? &s2 : nullptr, stream, ws_mode, ws_offset + (ws_mode == WS_STATIC ? total : 0));
  if (pooled) (void)hipFreeAsync(ws, hs);  // back to the pool once the kernels have run
  if (st != THL_OK) return st;
  std::snprintf(t_staged_name, sizeof(t_staged_name), "%s+cvt_%s", t_last_variant,
                sg.a && sg.b ? "ab" : (sg.a ? "a" : "b"));
  t_last_variant = t_staged_name;
  return THL_OK;
}

// Grouped problems: each validated as by thl_gemm, then checked against each
// other, and run with one variant, grid row z computing problem z from the
// device copy of the descriptors.
thl_status grouped_impl(int64_t count, const thl_group_problem* pb, const thl_group_problem* pb_dev, thl_op opA,
                        thl_op opB, float alpha, float beta, const thl_dtypes* dt, const thl_epilogue* epi,
                        const thl_scales* sc, struct ihipStream_t* stream) {
  if (count < 0 || !dt) return THL_ERR_INVALID;
  if (count > 65535) return THL_ERR_UNSUPPORTED;  // one grid row per problem
  if (count > 0 && !pb) return THL_ERR_INVALID;
  if (is_mx_out(dt->d)) return THL_ERR_UNSUPPORTED;  // MX output: single problems only
  const unsigned flags = epi ? epi->flags : 0u;
  const Batch one{};
  std::vector<Prep> preps(static_cast<size_t>(count));
  int64_t tiles_256 = 0, tiles_128 = 0;
  bool any_work = false, all_vec = true;
  int64_t ref = -1;  // the first problem with outputs: its family is the group's
  for (int64_t z = 0; z < count; ++z) {
    const thl_group_problem& q = pb[z];
    thl_scales s = sc ? *sc : thl_scales{1.0f, 1.0f, nullptr, 0, nullptr, 0};
    s.sfa = q.sfa;
    s.ld_sfa = q.ld_sfa;
    s.sfb = q.sfb;
    s.ld_sfb = q.ld_sfb;
    const thl_status st = prepare(one, q.m, q.n, q.k, q.A, q.lda, opA, q.B, q.ldb, opB, q.C, q.ldc, q.D, q.ldd,
                                  alpha, beta, dt, flags, q.bias, &s, nullptr, 0, &preps[z]);
    if (st != THL_OK) return st;
    if (preps[z].work) {
      // one family for the problems with outputs: block scales on every one
      // of them or on none
      if (ref < 0) ref = z;
      if (preps[z].fam != preps[ref].fam) return THL_ERR_INVALID;
      any_work = true;
      all_vec = all_vec && preps[z].vec;
      tiles_256 += ((q.m + 255) / 256) * ((q.n + 255) / 256);
      tiles_128 += ((q.m + 127) / 128) * ((q.n + 127) / 128);
    }
  }
  if (count == 0) return THL_OK;
  if (any_work && !pb_dev) return THL_ERR_INVALID;

  // ---- no problem's D overlaps another problem's D or anything it reads
  if (any_work) {
    struct Span {
      Range r;
      int64_t z;
      bool is_d;
    };
    std::vector<Span> spans;
    for (int64_t z = 0; z < count; ++z) {
      const thl_group_problem& q = pb[z];
      const Prep& pr = preps[z];
      if (!pr.work) continue;
      const int64_t ra = opA == THL_OP_N ? q.m : q.k, ca = opA == THL_OP_N ? q.k : q.m;
      const int64_t rb = opB == THL_OP_N ? q.k : q.n, cb = opB == THL_OP_N ? q.n : q.k;
      spans.push_back({matrix_range(q.D, dt->d, q.m, q.n, q.ldd), z, true});
      if (q.k > 0) {
        spans.push_back({matrix_range(q.A, dt->a, ra, ca, q.lda), z, false});
        spans.push_back({matrix_range(q.B, dt->b, rb, cb, q.ldb), z, false});
      }
      if (beta != 0.0f) spans.push_back({matrix_range(q.C, dt->c, q.m, q.n, q.ldc), z, false});
      if (pr.has_bias) spans.push_back({matrix_range(q.bias, dt->bias, q.m, 1, q.m), z, false});
      if (pr.block_scaled && q.k > 0) {
        spans.push_back({matrix_range(q.sfa, THL_E8M0, q.k / 32, q.m, q.ld_sfa), z, false});
        spans.push_back({matrix_range(q.sfb, THL_E8M0, q.k / 32, q.n, q.ld_sfb), z, false});
      }
    }
    // D spans sorted by start: neighbours must not overlap, and every other
    // span of another problem must miss them all (its own problem's spans
    // were checked by prepare; C == D of one problem is its exact alias).
    std::vector<Span> ds;
    for (const Span& sp : spans)
      if (sp.is_d && sp.r.lo < sp.r.hi) ds.push_back(sp);
    std::sort(ds.begin(), ds.end(), [](const Span& a, const Span& b) { return a.r.lo < b.r.lo; });
    for (size_t i = 1; i < ds.size(); ++i)
      if (ds[i].r.lo < ds[i - 1].r.hi) return THL_ERR_INVALID;
    for (const Span& sp : spans) {
      if (sp.is_d || sp.r.lo >= sp.r.hi) continue;
      // first D span ending after sp starts
      auto it = std::upper_bound(ds.begin(), ds.end(), sp.r.lo,
                                 [](uintptr_t v, const Span& d) { return v < d.r.hi; });
      for (; it != ds.end() && it->r.lo < sp.r.hi; ++it)
        if (it->z != sp.z) return THL_ERR_INVALID;
    }
  }

  // ---- one variant for every problem (tiled kernels only)
  thl_status st = THL_OK;
  const Prep& pref = preps[ref < 0 ? 0 : ref];
  const int want = want_tier_of(tiles_256, tiles_128);
  const int ncu = cu_count();
  const Variant* pick = choose_variant(pref, false, 0, want, want == 2 && ncu > 0 && tiles_128 <= ncu,
                                       [&](const Variant& v) {
                                         for (int64_t z = 0; z < count; ++z)
                                           if (preps[z].work && !fits(v, preps[z], one, pb[z].A, pb[z].B, pb[z].k))
                                             return false;
                                         return true;
                                       },
                                       &st);
  if (!pick) return st;
  if (!any_work) {
    t_last_variant = pick->name;
    return THL_OK;
  }
  int64_t max_tiles = 0;
  for (int64_t z = 0; z < count; ++z) {
    const int64_t t = preps[z].work ? ((pb[z].m + pick->bm - 1) / pick->bm) * ((pb[z].n + pick->bn - 1) / pick->bn) : 0;
    if (t > INT32_MAX) return THL_ERR_UNSUPPORTED;
    max_tiles = t > max_tiles ? t : max_tiles;
  }
  // Group-wide arguments; the kernel fills in each row's problem from the
  // device descriptors.
  Prep p0 = pref;
  p0.vec = all_vec;
  GemmArgs a = make_args(p0, *pick, 0, 0, 0, nullptr, nullptr, nullptr, 0, nullptr, 0, alpha, beta, dt, nullptr);
  a.group = reinterpret_cast<const GroupProblem*>(pb_dev);
  a.elem_bits_a = static_cast<int32_t>(dt->a == THL_E2M1X2 ? 4 : 8 * bytes_of(dt->a, 1));
  a.elem_bits_b = static_cast<int32_t>(dt->b == THL_E2M1X2 ? 4 : 8 * bytes_of(dt->b, 1));
  const int64_t grid = persistent_grid(*pick, count, max_tiles);
  if (grid <= 0) return THL_ERR_HIP;
  a.xcd_local = count % 8 == 0 ? 1 : 0;
  if (pick->launch(a, dim3(static_cast<unsigned>(count), static_cast<unsigned>(grid)),
                   reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return THL_ERR_HIP;
  t_last_variant = pick->name;
  last_splits = 1;
  return THL_OK;
}

}  // namespace
}  // namespace thl

// The no-allocation entry point's scratch: the split-K partial matrices.  The
// split rule bounds them by splits * tiles * 128 * 128 * 4 bytes with
// splits * tiles at most the 512 resident 128x128 workgroups, i.e. 32 MiB plus
// the rounding of m to 4 rows and of each split to 256 bytes; 40 MiB holds
// every split thl_gemm would choose.  Each GPU keeps its copy until the
// process ends.
static constexpr int64_t kScratchBytes = INT64_C(40) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace thl {
namespace {

// The scratch array's device address on each device, read once per device
// (with that device current) at its first no-allocation call.  In host code
// the array's name is only a stand-in: kernels get this address.
std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[64];

thl_status static_scratch(hipStream_t, int64_t bytes, uint8_t** out) {
  if (bytes > kScratchBytes) return THL_ERR_SCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return THL_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return THL_ERR_HIP;
    }
    g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return THL_OK;
}

}  // namespace
}  // namespace thl

extern "C" {

// ---------------------------------------------------------------- index maps

const char* thl_kernel_index_map_names(void) {
  return "xcd_remap,grouped_tile,swz,lds_offset,copy_source,mfma32_operand,mfma32_acc,fp8_32x32_k,tr16_source,"
         "mm_lds_offset,mm_copy_source,tr16_operand,pair_lds_offset,pair_copy_source,mfma16_operand,mfma16_acc";
}

int thl_kernel_index_map(const char* map, const int64_t* params, int64_t n, const int64_t* in, int64_t* out) {
  if (!map || n < 0 || (n > 0 && (!in || !out))) return THL_ERR_INVALID;
  auto param = [&](int i) { return params ? params[i] : 0; };
  for (int64_t t = 0; t < n; ++t) {
    const int64_t x = in[2 * t], y = in[2 * t + 1];
    int64_t r0 = 0, r1 = 0;
    if (!std::strcmp(map, "xcd_remap")) {
      if (!params || param(0) <= 0) return THL_ERR_INVALID;
      r0 = maps::xcd_remap(x, param(0));
    } else if (!std::strcmp(map, "grouped_tile")) {
      if (!params || param(0) <= 0 || param(1) <= 0 || param(2) <= 0) return THL_ERR_INVALID;
      maps::grouped_tile(x, param(0), param(1), param(2), &r0, &r1);
    } else if (!std::strcmp(map, "swz")) {
      r0 = maps::swz(x);
    } else if (!std::strcmp(map, "lds_offset")) {
      r0 = maps::lds_offset(x, y);
    } else if (!std::strcmp(map, "copy_source")) {
      if (!params || (param(0) != 4 && param(0) != 16)) return THL_ERR_INVALID;
      maps::copy_source(x, y, param(0), &r0, &r1);
    } else if (!std::strcmp(map, "mfma32_operand")) {
      if (!params || param(0) <= 0) return THL_ERR_INVALID;
      maps::mfma32_operand(x, y, param(0), &r0, &r1);
    } else if (!std::strcmp(map, "mfma32_acc")) {
      maps::mfma32_acc(x, y, &r0, &r1);
    } else if (!std::strcmp(map, "fp8_32x32_k")) {
      r0 = maps::fp8_32x32_k_of(x, y);
    } else if (!std::strcmp(map, "tr16_source")) {
      maps::tr16_source(x, y, &r0, &r1);
    } else if (!std::strcmp(map, "mm_lds_offset")) {
      if (!params || param(0) <= 0 || param(0) % 256 != 0) return THL_ERR_INVALID;
      r0 = maps::mm_lds_offset(x, y, param(0));
    } else if (!std::strcmp(map, "mm_copy_source")) {
      if (!params || (param(0) != 4 && param(0) != 16) || param(1) <= 0 || param(1) % 256 != 0) return THL_ERR_INVALID;
      maps::mm_copy_source(x, y, param(0), param(1), &r0, &r1);
    } else if (!std::strcmp(map, "tr16_operand")) {
      maps::tr16_operand(x, y, &r0, &r1);
    } else if (!std::strcmp(map, "pair_lds_offset")) {
      if (!params || (param(0) != 0 && param(0) != 1)) return THL_ERR_INVALID;
      r0 = maps::pair_lds_offset(x, y, param(0));
    } else if (!std::strcmp(map, "pair_copy_source")) {
      maps::pair_copy_source(x, y, &r0, &r1);
    } else if (!std::strcmp(map, "mfma16_operand")) {
      maps::mfma16_operand(x, y, &r0, &r1);
    } else if (!std::strcmp(map, "mfma16_acc")) {
      maps::mfma16_acc(x, y, &r0, &r1);
    } else {
      return THL_ERR_INVALID;
    }
    out[2 * t] = r0;
    out[2 * t + 1] = r1;
  }
  return THL_OK;
}

}  // extern "C"
