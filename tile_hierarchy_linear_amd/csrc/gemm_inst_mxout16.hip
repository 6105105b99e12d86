// MX-output variants (D as MX blocks with generated scales) of the 16-bit
// families, every operand orientation.
#include "gemm_launch.hpp"

using thl::GemmArgs;
using thl::FAM_BF16;
using thl::FAM_F16;

THL_INST_MXOUT(FAM_BF16, true, true)
THL_INST_MXOUT(FAM_BF16, false, true)
THL_INST_MXOUT(FAM_BF16, true, false)
THL_INST_MXOUT(FAM_BF16, false, false)
THL_INST_MXOUT(FAM_F16, true, true)
THL_INST_MXOUT(FAM_F16, false, true)
THL_INST_MXOUT(FAM_F16, true, false)
THL_INST_MXOUT(FAM_F16, false, false)
