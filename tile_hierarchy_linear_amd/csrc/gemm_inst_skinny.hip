// The small-M kernel for every operand family with K-major A and B (4
// wavefronts splitting K; 1, 2 or 4 sixteen-row tiles) and its launcher.
#include "gemm_args.hpp"
#include "gemm_skinny.hpp"

namespace thl {

template <int F, int KW, int MT>
hipError_t launch_skinny(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  GemmArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&skinny_kernel<F, KW, 2, MT>), grid, dim3(KW * 64), args, 0,
                         stream);
}

#define THL_SKINNY(F)                                                               \
  template hipError_t launch_skinny<F, 4, 1>(const GemmArgs&, dim3, hipStream_t); \
  template hipError_t launch_skinny<F, 4, 2>(const GemmArgs&, dim3, hipStream_t); \
  template hipError_t launch_skinny<F, 4, 4>(const GemmArgs&, dim3, hipStream_t);

THL_SKINNY(FAM_BF16)
THL_SKINNY(FAM_F16)
THL_SKINNY(FAM_I8)
THL_SKINNY(FAM_FP8)
THL_SKINNY(FAM_E5M2)
THL_SKINNY(FAM_E4E5)
THL_SKINNY(FAM_E5E4)
THL_SKINNY(FAM_FP4)

}  // namespace thl
