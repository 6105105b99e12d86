// Kernel instantiations for MXFP8 with E5M2 elements (E8M0 block scales),
// K-major operands.
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_MX8_E5M2;

THL_INSTANTIATE_VARIANTS_MX8(FAM_MX8_E5M2)
