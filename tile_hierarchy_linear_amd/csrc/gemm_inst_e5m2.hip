// Kernel instantiations for the e5m2 operand family, K-major operands
// (one unit per family so the library builds in parallel).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_E5M2;

THL_INSTANTIATE_VARIANTS(FAM_E5M2, true, true)
