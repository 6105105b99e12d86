// gemm_launch.hpp -- definition of the variant launcher; included by the
// per-family instantiation units only.
#pragma once

#include "gemm_args.hpp"
#include "gemm_kernels.hpp"

namespace thl {

// hipLaunchKernel reports this launch's own status (a stale error left by
// an unrelated earlier HIP call in the process is not picked up).
template <int F, int BM, int BN, int WM, int WN, int LOADW, int STAGES, int OCC, int SCW>
hipError_t launch_kmajor(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  GemmArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&gemm_kmajor_kernel<F, BM, BN, WM, WN, LOADW, STAGES, OCC, SCW>), grid,
      dim3(WM * WN * 64), args, 0, stream);
}

}  // namespace thl

// The variants built for one family (used by each instantiation unit and,
// as names, by the dispatch table).
#define THL_INSTANTIATE_KMAJOR(FAM, SCW)                                                                     \
  template hipError_t thl::launch_kmajor<FAM, 256, 256, 2, 2, 16, 4, 1, SCW>(const GemmArgs&, dim3, hipStream_t); \
  template hipError_t thl::launch_kmajor<FAM, 256, 128, 2, 2, 16, 3, 2, SCW>(const GemmArgs&, dim3, hipStream_t); \
  template hipError_t thl::launch_kmajor<FAM, 128, 128, 2, 2, 16, 4, 2, SCW>(const GemmArgs&, dim3, hipStream_t); \
  template hipError_t thl::launch_kmajor<FAM, 128, 128, 2, 2, 4, 4, 2, SCW>(const GemmArgs&, dim3, hipStream_t);
