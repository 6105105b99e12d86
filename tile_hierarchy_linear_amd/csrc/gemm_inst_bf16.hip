// Kernel instantiations for the bf16 operand family, K-major operands
// (one unit per family so the library builds in parallel).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_BF16;

THL_INSTANTIATE_VARIANTS(FAM_BF16, true, true)
