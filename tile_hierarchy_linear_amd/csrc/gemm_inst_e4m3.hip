// Kernel instantiations for the e4m3 operand family, K-major operands
// (one unit per family so the library builds in parallel).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_FP8;

THL_INSTANTIATE_VARIANTS(FAM_FP8, true, true)
