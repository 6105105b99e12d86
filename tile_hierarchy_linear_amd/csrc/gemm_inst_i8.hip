// Kernel instantiations for the i8 operand family, K-major operands
// (one unit per family so the library builds in parallel).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_I8;

THL_INSTANTIATE_VARIANTS(FAM_I8, true, true)
