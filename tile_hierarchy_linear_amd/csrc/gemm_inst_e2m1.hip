// Kernel instantiations for the e2m1 operand family, K-major operands
// (one unit per family so the library builds in parallel).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_FP4;

THL_INSTANTIATE_VARIANTS_FP4()
