// Kernel instantiations for MXFP8 (e4m3 with E8M0 block scales), K-major
// operands (one unit per family so the library builds in parallel).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_MX8;

THL_INSTANTIATE_VARIANTS_MX8(FAM_MX8)
