// convert.hpp -- the operand conversion pass (convert.hip): a narrow operand
// rewritten as K-major rows the tiled GEMM kernels stage directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace thl {

struct CvtArgs {
  const uint8_t* src;  // the operand as the caller stores it (first problem)
  int64_t ld_bytes;    // bytes from one source line to the next
  int64_t line_bytes;  // bytes a line holds data in: ceil(line length * bits / 8)
  int64_t src_batch;   // bytes from one problem's operand to the next
  int32_t src_fmt;     // thl_dtype of the stored elements
  int32_t dst_fmt;     // THL_E4M3 (widened), or src_fmt (moved as it is)
  int32_t kmajor;      // 1: line r is logical row r (contiguous along K); 0: line p is K-index p
  int32_t aligned4;    // source base, ld_bytes and src_batch are multiples of 4 bytes
  int64_t rows, k;     // the logical operand: rows x k (rows = m for A, n for B)
  uint8_t* dst;        // row r of the output at dst + r * dst_ld_bytes, 16-byte aligned
  int64_t dst_ld_bytes;  // a multiple of 64; bytes past K are written as zeros
  int64_t dst_batch;     // bytes from one problem's output to the next
};

// Launches the pass over `batch` problems on stream s.  hipErrorInvalidValue
// for a combination it does not build or a grid beyond its limits (rows up
// to 65535 tiles of 64 for K-major sources, of 256 otherwise; batch up to
// 65535).
hipError_t launch_convert(const CvtArgs& a, int64_t batch, hipStream_t s);

}  // namespace thl
