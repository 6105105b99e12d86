// Kernel instantiations for mixed fp8 operands (e5m2 A with e4m3 B), K-major operands
// (one unit per family so the library builds in parallel).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_E5E4;

THL_INSTANTIATE_VARIANTS(FAM_E5E4, true, true)
