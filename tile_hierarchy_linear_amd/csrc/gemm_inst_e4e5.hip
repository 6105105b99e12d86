// Kernel instantiations for mixed fp8 operands (e4m3 A with e5m2 B), K-major operands
// (one unit per family so the library builds in parallel).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_E4E5;

THL_INSTANTIATE_VARIANTS(FAM_E4E5, true, true)
