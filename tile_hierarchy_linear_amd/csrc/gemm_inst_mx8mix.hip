// Kernel instantiations for MXFP8 with E4M3 A and E5M2 B, and the other
// way round (E8M0 block scales), K-major operands.
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_MX8_E4E5;
using thl::FAM_MX8_E5E4;

THL_INSTANTIATE_VARIANTS_MX8(FAM_MX8_E4E5)
THL_INSTANTIATE_VARIANTS_MX8(FAM_MX8_E5E4)
