// convert.hip -- rewrites a narrow operand as K-major rows for the tiled
// GEMM kernels.
//
// The tiled kernels stage operand rows of 64 bytes of K straight from global
// memory into LDS.  An 8-bit operand stored along M (N), or a 6-bit operand
// (four elements in three bytes, which no 64-byte step holds whole), or a
// 4-bit operand beside another format, is first rewritten here: rows of the
// logical operand (A: m rows, B: n columns) become contiguous along K, in
// the same 8-bit format, as E2M1 pairs when both operands are E2M1, or
// widened to E4M3.  The widening is exact: every E2M1, E2M3 and E3M2 value is
// an E4M3 value (their exponent ranges, 2^0..2^2, 2^-3..2^2 with subnormals,
// 2^-4..2^4, lie inside E4M3's 2^-9..2^8, and their 1, 3 and 2 mantissa bits
// inside its 3).  Block scales are indexed by (row, K/32) whatever the
// storage, so they apply unchanged to the rewritten operand.  The formats are
// those of the "Blackwell Narrow Precision Data Types" table ("Technical
// Documentation: NVIDIA/cutlass", "Blackwell SM100 GEMMs"), which also lists
// every pairing of them in all four layouts ("Layouts, Tensor Alignment
// Requirements to Target tcgen05.mma Instructions", Tables 2 and 3).
//
// One workgroup of 256 lanes writes one 64-row x 64-byte tile of the output
// (64 K-elements of 8 bits, or 128 of 4 bits): it reads the tile's source
// elements along the source's contiguous dimension (16 or 32 consecutive
// elements a lane), converts each to its output code in registers, parks
// the codes in LDS as a [row][k] byte array, and writes each output row
// segment as one 16-byte store.  The pass is bound by HBM: per element it
// reads bits/8 bytes and writes one byte (half a byte for E2M1 output).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/thl.h"
#include "convert.hpp"

namespace thl {
namespace {

constexpr int kRows = 64;  // output rows per tile

// E4M3 code of an E2M1 code (1 sign, 2 exponent bits with bias 1, 1 mantissa
// bit): 0.5 (the one subnormal) is 2^-1, exponent field 6; a normal code with
// exponent e and mantissa f is 2^(e-1) (1 + f/2), exponent field e + 6 and
// mantissa f * 4.
__device__ __forceinline__ uint32_t e4m3_of_e2m1(uint32_t c) {
  const uint32_t s = (c & 8u) << 4, e = (c >> 1) & 3u, f = c & 1u;
  uint32_t mag;
  if (e != 0)
    mag = ((e + 6u) << 3) | (f << 2);
  else
    mag = f ? (6u << 3) : 0u;
  return s | mag;
}

// E4M3 code of an E2M3 code (1 sign, 2 exponent bits with bias 1, 3 mantissa
// bits).  Normal: 2^(e-1) (1 + f/8) has exponent field e + 6 and the same
// mantissa.  Subnormal f/8 (f = 1 .. 7): with h the top set bit of f, the
// value is 2^(h-3) (1 + rest/2^h), exponent field h + 4 and mantissa
// f << (3 - h) without its leading bit.
__device__ __forceinline__ uint32_t e4m3_of_e2m3(uint32_t c) {
  const uint32_t s = (c & 32u) << 2, e = (c >> 3) & 3u, f = c & 7u;
  uint32_t mag;
  if (e != 0) {
    mag = ((e + 6u) << 3) | f;
  } else if (f == 0) {
    mag = 0;
  } else {
    const uint32_t h = 31u - static_cast<uint32_t>(__builtin_clz(f));
    mag = ((h + 4u) << 3) | ((f << (3u - h)) & 7u);
  }
  return s | mag;
}

// E4M3 code of an E3M2 code (1 sign, 3 exponent bits with bias 3, 2 mantissa
// bits).  Normal: 2^(e-3) (1 + f/4) has exponent field e + 4 and mantissa
// f * 2.  Subnormal f/4 * 2^-2 = f * 2^-4 (f = 1 .. 3): with h the top set
// bit of f, exponent field h + 3 and mantissa f << (3 - h) without its
// leading bit.
__device__ __forceinline__ uint32_t e4m3_of_e3m2(uint32_t c) {
  const uint32_t s = (c & 32u) << 2, e = (c >> 2) & 7u, f = c & 3u;
  uint32_t mag;
  if (e != 0) {
    mag = ((e + 4u) << 3) | (f << 1);
  } else if (f == 0) {
    mag = 0;
  } else {
    const uint32_t h = 31u - static_cast<uint32_t>(__builtin_clz(f));
    mag = ((h + 3u) << 3) | ((f << (3u - h)) & 7u);
  }
  return s | mag;
}

template <int SRC, int DST>
__device__ __forceinline__ uint32_t out_code(uint32_t c) {
  if constexpr (DST == THL_E4M3 && SRC == THL_E2M1X2) return e4m3_of_e2m1(c);
  if constexpr (DST == THL_E4M3 && SRC == THL_E2M3) return e4m3_of_e2m3(c);
  if constexpr (DST == THL_E4M3 && SRC == THL_E3M2) return e4m3_of_e3m2(c);
  return c;  // same format: the code moves as it is
}

template <int SRC>
constexpr int bits_of_fmt() {
  return SRC == THL_E2M1X2 ? 4 : ((SRC == THL_E2M3 || SRC == THL_E3M2) ? 6 : 8);
}

// E elements of one source line from element e0 on: the covering bytes as
// 32-bit words (4-byte loads when the line is 4-byte aligned and the span
// lies inside it, byte loads otherwise; bytes past the line read as 0).
template <int NW>
__device__ __forceinline__ void fetch_words(const uint8_t* line, int64_t start, int64_t line_bytes, bool aligned4,
                                            uint32_t (&w)[NW]) {
  if (aligned4 && start + 4 * NW <= line_bytes) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(line + start);
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = __builtin_nontemporal_load(p + i);
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t at = start + 4 * i + b;
        if (at < line_bytes) v |= static_cast<uint32_t>(line[at]) << (8 * b);
      }
      w[i] = v;
    }
  }
}

// Code of element i (bits BITS each, little-endian bit order) of the words.
template <int BITS, int NW>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[NW], int i) {
  const int bit = i * BITS;
  const int wi = bit >> 5, sh = bit & 31;
  uint32_t v = w[wi] >> sh;
  if constexpr (BITS == 6) {
    if (sh > 26 && wi + 1 < NW) v |= w[wi + 1] << (32 - sh);
  }
  return v & ((1u << BITS) - 1u);
}

template <int SRC, int DST>
__global__ void __launch_bounds__(256) convert_kernel(CvtArgs p) {
  constexpr int BITS = bits_of_fmt<SRC>();
  constexpr int KT = DST == THL_E2M1X2 ? 128 : 64;  // K-elements per tile (64 output bytes a row)
  constexpr int E = KT / 4;                          // elements a lane reads
  constexpr int NW = E * BITS / 32;                  // their words
  constexpr int PITCH = KT + 4;                      // LDS row pitch (bytes)
  __shared__ uint8_t tile[kRows * PITCH];

  const int t = static_cast<int>(threadIdx.x);
  const int64_t z = blockIdx.z;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kRows;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * KT;
  const uint8_t* src = p.src + z * p.src_batch;

  // ---- read and convert
  if (p.kmajor) {
    // line = row r0 + t/4, elements p0 + E*(t%4) ..
    const int r = t >> 2, seg = t & 3;
    const int64_t row = r0 + r, e0 = p0 + E * seg;
    uint32_t w[NW];
    if (row < p.rows) {
      fetch_words<NW>(src + row * p.ld_bytes, e0 * BITS / 8, p.line_bytes, p.aligned4 != 0, w);
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) w[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t c = (e0 + i < p.k) ? out_code<SRC, DST>(code_at<BITS, NW>(w, i)) : 0u;
      tile[r * PITCH + E * seg + i] = static_cast<uint8_t>(c);
    }
  } else {
    // line = k-index p0 + col, elements (rows) r0 + E*rseg ..
    constexpr int PER_COL = 256 / KT;  // lanes per source line
    const int col = t / PER_COL, rseg = t % PER_COL;
    const int64_t kk = p0 + col, e0 = r0 + E * rseg;
    uint32_t w[NW];
    if (kk < p.k) {
      fetch_words<NW>(src + kk * p.ld_bytes, e0 * BITS / 8, p.line_bytes, p.aligned4 != 0, w);
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) w[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t c = (e0 + i < p.rows) ? out_code<SRC, DST>(code_at<BITS, NW>(w, i)) : 0u;
      tile[(E * rseg + i) * PITCH + col] = static_cast<uint8_t>(c);
    }
  }
  __syncthreads();

  // ---- write: lane t stores 16 bytes of row t/4 (zeros past K)
  const int r = t >> 2, chunk = t & 3;
  const int64_t row = r0 + r;
  if (row >= p.rows) return;
  uint32_t o[4];
  if constexpr (DST == THL_E2M1X2) {
    // 32 codes, two a byte, the even element in the low nibble
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) v |= static_cast<uint32_t>(tile[r * PITCH + 32 * chunk + 8 * q + b] & 15u) << (4 * b);
      o[q] = v;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) v |= static_cast<uint32_t>(tile[r * PITCH + 16 * chunk + 4 * q + b]) << (8 * b);
      o[q] = v;
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(p.dst + z * p.dst_batch + row * p.dst_ld_bytes + blockIdx.x * 64 + 16 * chunk);
  *dst = make_uint4(o[0], o[1], o[2], o[3]);
}

template <int SRC, int DST>
hipError_t launch(const CvtArgs& a, int64_t batch, hipStream_t s) {
  constexpr int KT = DST == THL_E2M1X2 ? 128 : 64;
  (void)KT;
  const dim3 grid(static_cast<unsigned>(a.dst_ld_bytes / 64), static_cast<unsigned>((a.rows + kRows - 1) / kRows),
                  static_cast<unsigned>(batch));
  hipLaunchKernelGGL((convert_kernel<SRC, DST>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_convert(const CvtArgs& a, int64_t batch, hipStream_t s) {
  if (a.rows <= 0 || batch <= 0 || a.dst_ld_bytes <= 0 || a.dst_ld_bytes % 64 != 0) return hipErrorInvalidValue;
  if (a.dst_ld_bytes / 64 > INT32_MAX || (a.rows + kRows - 1) / kRows > 65535 || batch > 65535)
    return hipErrorInvalidValue;
  switch (a.src_fmt) {
    case THL_I8:
      return launch<THL_I8, THL_I8>(a, batch, s);
    case THL_E4M3:
      return launch<THL_E4M3, THL_E4M3>(a, batch, s);
    case THL_E5M2:
      return launch<THL_E5M2, THL_E5M2>(a, batch, s);
    case THL_E2M3:
      return launch<THL_E2M3, THL_E4M3>(a, batch, s);
    case THL_E3M2:
      return launch<THL_E3M2, THL_E4M3>(a, batch, s);
    case THL_E2M1X2:
      return a.dst_fmt == THL_E2M1X2 ? launch<THL_E2M1X2, THL_E2M1X2>(a, batch, s)
                                     : launch<THL_E2M1X2, THL_E4M3>(a, batch, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace thl
