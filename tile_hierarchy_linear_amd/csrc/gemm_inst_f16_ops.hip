// Kernel instantiations for the f16 operand family with an M-major A
// and/or an N-major B (opA = N, opB = T).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_F16;

THL_INSTANTIATE_VARIANTS(FAM_F16, false, true)
THL_INSTANTIATE_VARIANTS(FAM_F16, true, false)
THL_INSTANTIATE_VARIANTS(FAM_F16, false, false)
