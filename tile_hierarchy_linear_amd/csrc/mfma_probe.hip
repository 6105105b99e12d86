// mfma_probe.hip -- a matrix-core-only loop, for measurement: how many
// TFLOP/s the MFMA pipes deliver on this chip when they do nothing else, at
// the clock the chip holds under that load.  It moves no memory in its loop,
// so it is the ceiling the GEMM kernels could reach with the same
// instructions; the gap between it and the published dense peak is the
// clock.  Built as its own library (libthl_probe.so), outside the GEMM
// boundary.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;  // independent accumulators per wave: enough to issue back to back

// fmt 0: v_mfma_f32_32x32x16_bf16; 1: the f8f6f4 instruction on e4m3 (format
// 0, unscaled); 2: the same instruction on e2m1 with E8M0 scales (format 4).
template <int FMT>
__global__ void __launch_bounds__(256) mfma_loop(int64_t iters, float* out) {
  v16f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16f{};
  const int lane = static_cast<int>(threadIdx.x);
  // operands from the lane index, opaque to the compiler so the loop stays
  const int seed = __builtin_amdgcn_readfirstlane(lane) + lane;
  v8i a = {seed, seed + 1, seed + 2, seed + 3, seed + 4, seed + 5, seed + 6, seed + 7};
  v8i b = a + 9;
  a &= 0x3C3C3C3C;  // small finite codes in every format
  b &= 0x3C3C3C3C;
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if constexpr (FMT == 0) {
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, __builtin_shufflevector(a, a, 0, 1, 2, 3)),
                                                         __builtin_bit_cast(v8bf, __builtin_shufflevector(b, b, 0, 1, 2, 3)),
                                                         acc[c], 0, 0, 0);
      } else if constexpr (FMT == 1) {
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
      } else {
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 4, 4, 0, 127, 0, 127);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Launches `workgroups` workgroups of 256 lanes (four waves), each wave
// issuing iters x 8 MFMAs of format fmt (0 bf16, 1 e4m3, 2 e2m1 scaled) on
// `stream`; out receives one float per lane (workgroups x 256, device).
// Returns 0, or -1 for a bad argument or launch.  Flops per launch:
// workgroups x 4 x iters x 8 x (32768 for bf16, 131072 for e4m3 and e2m1).
int thl_probe_mfma(int fmt, int64_t iters, int workgroups, float* out, hipStream_t stream) {
  if (fmt < 0 || fmt > 2 || iters <= 0 || workgroups <= 0 || !out) return -1;
  const dim3 grid(static_cast<unsigned>(workgroups)), block(256);
  if (fmt == 0)
    hipLaunchKernelGGL(mfma_loop<0>, grid, block, 0, stream, iters, out);
  else if (fmt == 1)
    hipLaunchKernelGGL(mfma_loop<1>, grid, block, 0, stream, iters, out);
  else
    hipLaunchKernelGGL(mfma_loop<2>, grid, block, 0, stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
