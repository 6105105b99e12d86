// Kernel instantiations for the f16 operand family, K-major operands
// (one unit per family so the library builds in parallel).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_F16;

THL_INSTANTIATE_VARIANTS(FAM_F16, true, true)
