// gemm_launch.hpp -- definition of the variant launcher; included by the
// per-family instantiation units only.
#pragma once

#include "gemm_args.hpp"
#include "gemm_kernels.hpp"

namespace thl {

// hipLaunchKernel reports this launch's own status (a stale error left by
// an unrelated earlier HIP call in the process is not picked up).
template <int F, int BM, int BN, int WM, int WN, int LOADW, int STAGES, int OCC, int SCW, bool AK, bool BK, bool MXO>
hipError_t launch_gemm(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  GemmArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&gemm_kernel<F, BM, BN, WM, WN, LOADW, STAGES, OCC, SCW, AK, BK, MXO>), grid,
      dim3(WM * WN * 64), args, 0, stream);
}

}  // namespace thl

// The variants built for one family and operand orientation (used by each
// instantiation unit; the dispatch table lists the same set).
#define THL_INST(FAM, BM, BN, LOADW, ST, OCC, AK, BK) \
  template hipError_t thl::launch_gemm<FAM, BM, BN, 2, 2, LOADW, ST, OCC, 16, AK, BK, false>(const GemmArgs&, dim3, \
                                                                                            hipStream_t);

// The MX-output variant of a family and orientation: 128x128, 16-byte copies,
// two workgroups per CU.
#define THL_INST_MXOUT(FAM, AK, BK) \
  template hipError_t thl::launch_gemm<FAM, 128, 128, 2, 2, 16, 4, 2, 16, AK, BK, true>(const GemmArgs&, dim3, \
                                                                                       hipStream_t);

// fp4: no 256x128 three-stage variant (its K-step groups of four need a
// stage count that divides into them).
#define THL_INSTANTIATE_VARIANTS_FP4()                 \
  THL_INST(FAM_FP4, 256, 256, 16, 4, 1, true, true)    \
  THL_INST(FAM_FP4, 128, 128, 16, 4, 2, true, true)    \
  THL_INST(FAM_FP4, 128, 128, 4, 4, 2, true, true)

// MX fp8 families: as fp4 (scale groups of eight K-steps).
#define THL_INSTANTIATE_VARIANTS_MX8(FAM)       \
  THL_INST(FAM, 256, 256, 16, 4, 1, true, true) \
  THL_INST(FAM, 128, 128, 16, 4, 2, true, true) \
  THL_INST(FAM, 128, 128, 4, 4, 2, true, true)

#define THL_INSTANTIATE_VARIANTS(FAM, AK, BK) \
  THL_INST(FAM, 256, 256, 16, 4, 1, AK, BK)    \
  THL_INST(FAM, 256, 128, 16, 3, 2, AK, BK)    \
  THL_INST(FAM, 128, 128, 16, 6, 1, AK, BK)    \
  THL_INST(FAM, 128, 128, 16, 4, 2, AK, BK)    \
  THL_INST(FAM, 128, 128, 4, 4, 2, AK, BK)
