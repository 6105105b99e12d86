// The small-M kernel for every operand family (K-major A and B, 4 wavefronts
// splitting K) and its launcher.
#include "gemm_args.hpp"
#include "gemm_skinny.hpp"

namespace thl {

template <int F, int KW>
hipError_t launch_skinny(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  GemmArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&skinny_kernel<F, KW>), grid, dim3(KW * 64), args, 0, stream);
}

template hipError_t launch_skinny<FAM_BF16, 4>(const GemmArgs&, dim3, hipStream_t);
template hipError_t launch_skinny<FAM_F16, 4>(const GemmArgs&, dim3, hipStream_t);
template hipError_t launch_skinny<FAM_I8, 4>(const GemmArgs&, dim3, hipStream_t);
template hipError_t launch_skinny<FAM_FP8, 4>(const GemmArgs&, dim3, hipStream_t);
template hipError_t launch_skinny<FAM_E5M2, 4>(const GemmArgs&, dim3, hipStream_t);
template hipError_t launch_skinny<FAM_E4E5, 4>(const GemmArgs&, dim3, hipStream_t);
template hipError_t launch_skinny<FAM_E5E4, 4>(const GemmArgs&, dim3, hipStream_t);
template hipError_t launch_skinny<FAM_FP4, 4>(const GemmArgs&, dim3, hipStream_t);

}  // namespace thl
