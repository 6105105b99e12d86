// MX-output variants (D as MX blocks with generated scales) of the 8- and
// 4-bit families (K-major operands).
#include "gemm_launch.hpp"

using thl::GemmArgs;
using namespace thl;

THL_INST_MXOUT(FAM_FP8, true, true)
THL_INST_MXOUT(FAM_E5M2, true, true)
THL_INST_MXOUT(FAM_E4E5, true, true)
THL_INST_MXOUT(FAM_E5E4, true, true)
THL_INST_MXOUT(FAM_MX8, true, true)
THL_INST_MXOUT(FAM_MX8_E5M2, true, true)
THL_INST_MXOUT(FAM_MX8_E4E5, true, true)
THL_INST_MXOUT(FAM_MX8_E5E4, true, true)
THL_INST_MXOUT(FAM_FP4, true, true)
