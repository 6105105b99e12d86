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
// an E4M3 value (their exponent ranges, 2^-1..2^2, 2^-3..2^2 and 2^-4..2^4
// counting subnormals, lie inside E4M3's normal range 2^-6..2^8, and their
// 1, 3 and 2 mantissa bits inside its 3).  Block scales are indexed by (row, K/32) whatever the
// storage, so they apply unchanged to the rewritten operand.  The formats are
// those of the "Blackwell Narrow Precision Data Types" table ("Technical
// Documentation: NVIDIA/cutlass", "Blackwell SM100 GEMMs"), which also lists
// every pairing of them in all four layouts ("Layouts, Tensor Alignment
// Requirements to Target tcgen05.mma Instructions", Tables 2 and 3).
//
// One workgroup of 256 lanes writes one tile of the output: 64 rows x 256
// K-elements when the source is K-major, 256 rows x 128 (fp4: 256)
// K-elements when it is stored along the rows.  Consecutive lanes read
// consecutive chunks of one source line (128 to 256 contiguous bytes per
// line per wave instruction), convert each element to its output code in
// registers (an 8-bit source along the rows is turned around there in 4 x 16
// byte blocks), park the codes in LDS as a [row][k] byte array with 16-byte
// writes, and write the output rows in 16-byte stores, consecutive lanes
// along a row.
// The pass is bound by HBM: per element it reads bits/8 bytes and writes one
// byte (half a byte for E2M1 output).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/thl.h"
#include "convert.hpp"

namespace thl {
namespace {

// The value of a narrow code as an fp32, exactly: its magnitude bits go to
// the top of an fp32's exponent and mantissa fields (e exponent bits to the
// exponent field's low end, m mantissa bits to the mantissa's top), which
// reads as 2^(e-127) (1 + f/2^m), or for e = 0 as the fp32 subnormal
// f/2^m * 2^-126; one multiplication by 2^(127 - bias) rebases both to
// 2^(e-bias) (1 + f/2^m) and f/2^m * 2^(1-bias), the code's value.  E2M1:
// 2 exponent bits, bias 1; E2M3: 2 and bias 1; E3M2: 3 and bias 3.  The sign
// goes to bit 31.
template <int SRC>
__device__ __forceinline__ float narrow_value(uint32_t c) {
  if constexpr (SRC == THL_E2M1X2)
    return __builtin_bit_cast(float, ((c & 7u) << 22) | ((c & 8u) << 28)) * 0x1p126f;
  else if constexpr (SRC == THL_E2M3)
    return __builtin_bit_cast(float, ((c & 31u) << 20) | ((c & 32u) << 26)) * 0x1p126f;
  else
    return __builtin_bit_cast(float, ((c & 31u) << 21) | ((c & 32u) << 26)) * 0x1p124f;
}

// The output code of a source code: widened to E4M3 by the hardware's fp32 ->
// E4M3 conversion (exact here: every E2M1, E2M3 and E3M2 value is an E4M3
// value), or moved as it is.
template <int SRC, int DST>
__device__ __forceinline__ uint32_t out_code(uint32_t c) {
  if constexpr (DST == THL_E4M3 && SRC != THL_E4M3)
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(narrow_value<SRC>(c), 0.0f, 0, false)) & 255u;
  else
    return c;
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
    // one load of NW dwords (4-byte alignment is all a multi-dword global
    // load needs), so consecutive lanes read one contiguous run
    typedef uint32_t vec_t __attribute__((ext_vector_type(NW), aligned(4)));
    const vec_t x = __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(line + start));
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = x[i];
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

// Tile geometry: rows and K-elements per tile, and output bytes per tile row.
template <int DST, bool KMAJ>
struct Tile {
  static constexpr int ROWS = KMAJ ? 64 : 256;
  static constexpr int KT = KMAJ ? 256 : (DST == THL_E2M1X2 ? 256 : 128);
  static constexpr int OUT_BYTES = DST == THL_E2M1X2 ? KT / 2 : KT;
  static constexpr int PITCH = KT + 16;  // LDS row pitch: 16-byte aligned rows
};

// Four codes (bytes of the output format) into one word, the first lowest.
__device__ __forceinline__ uint32_t bytes4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

template <int SRC, int DST, bool KMAJ>
__global__ void __launch_bounds__(256) convert_kernel(CvtArgs p) {
  using G = Tile<DST, KMAJ>;
  constexpr int BITS = bits_of_fmt<SRC>();
  constexpr int E = 16;              // elements per chunk
  constexpr int NW = E * BITS / 32;  // words per chunk: 2, 3 or 4
  constexpr int PITCH = G::PITCH;
  __shared__ __attribute__((aligned(16))) uint8_t tile[G::ROWS * PITCH];

  const int t = static_cast<int>(threadIdx.x);
  const int64_t z = blockIdx.z;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * G::ROWS;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * G::KT;
  const uint8_t* src = p.src + z * p.src_batch;

  if constexpr (KMAJ) {
    // ---- K-major source: chunk q = t + 256 i is 16 elements of row q / 16;
    // the 16 codes go to LDS as one 16-byte write (a quarter-wave covers one
    // row's 256 bytes: every bank once)
    constexpr int CPL = G::KT / E;
#pragma unroll 2
    for (int i = 0; i < G::ROWS * CPL / 256; ++i) {
      const int q = t + 256 * i;
      const int ln = q / CPL, ch = q % CPL;
      const int64_t row = r0 + ln, e0 = p0 + E * ch;
      uint32_t w[NW];
      if (row < p.rows && e0 < p.k) {
        fetch_words<NW>(src + row * p.ld_bytes, e0 * BITS / 8, p.line_bytes, p.aligned4 != 0, w);
      } else {
#pragma unroll
        for (int j = 0; j < NW; ++j) w[j] = 0;
      }
      uint32_t o[4];
      const bool whole = e0 + E <= p.k;  // no element past K in this chunk
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if constexpr (DST == THL_E4M3 && SRC != THL_E4M3) {
          // four values, two per conversion instruction
          float v[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int j = 4 * h + b;
            v[b] = (whole || e0 + j < p.k) ? narrow_value<SRC>(code_at<BITS, NW>(w, j)) : 0.0f;
          }
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], x, true);
          o[h] = static_cast<uint32_t>(x);
        } else {
          uint32_t c[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int j = 4 * h + b;
            c[b] = (whole || e0 + j < p.k) ? code_at<BITS, NW>(w, j) : 0u;
          }
          o[h] = bytes4(c[0], c[1], c[2], c[3]);
        }
      }
      *reinterpret_cast<uint4*>(tile + ln * PITCH + E * ch) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else if constexpr (BITS == 8) {
    // ---- 8-bit source stored along the rows: lane l of wave v takes rows
    // 4l .. 4l+3 of 16 consecutive K-lines (one 4-byte load from each; a
    // wave reads 256 contiguous bytes of a line per instruction), turns the
    // 4 x 16 bytes around in registers, and writes its four rows' 16 codes
    // as 16-byte LDS writes (16 lanes cover 64 distinct banks)
    const int lane = t & 63, v = t >> 6;
    const int64_t row4 = r0 + 4 * lane;  // first of the lane's four rows
#pragma unroll 1
    for (int kg = v; kg < G::KT / 16; kg += 4) {
      uint32_t L[16];
#pragma unroll
      for (int l = 0; l < 16; ++l) {
        const int64_t kk = p0 + 16 * kg + l;
        uint32_t x = 0;
        if (kk < p.k) {
          const uint8_t* line = src + kk * p.ld_bytes;
          if (p.aligned4 && row4 + 4 <= p.rows) {
            x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(line + row4));
          } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
              if (row4 + b < p.rows) x |= static_cast<uint32_t>(line[row4 + b]) << (8 * b);
          }
        }
        L[l] = x;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          o[h] = bytes4((L[4 * h] >> (8 * i)) & 255u, (L[4 * h + 1] >> (8 * i)) & 255u,
                        (L[4 * h + 2] >> (8 * i)) & 255u, (L[4 * h + 3] >> (8 * i)) & 255u);
        *reinterpret_cast<uint4*>(tile + (4 * lane + i) * PITCH + 16 * kg) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  } else {
    // ---- 6- or 4-bit source stored along the rows: chunk q = t + 256 i is
    // 16 elements (rows) of K-line q / 16, written to LDS a byte at a time
    constexpr int CPL = G::ROWS / E;
#pragma unroll 2
    for (int i = 0; i < G::KT * CPL / 256; ++i) {
      const int q = t + 256 * i;
      const int ln = q / CPL, ch = q % CPL;
      const int64_t kk = p0 + ln, e0 = r0 + E * ch;
      uint32_t w[NW];
      if (kk < p.k && e0 < p.rows) {
        fetch_words<NW>(src + kk * p.ld_bytes, e0 * BITS / 8, p.line_bytes, p.aligned4 != 0, w);
      } else {
#pragma unroll
        for (int j = 0; j < NW; ++j) w[j] = 0;
      }
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const uint32_t c = (e0 + j < p.rows) ? out_code<SRC, DST>(code_at<BITS, NW>(w, j)) : 0u;
        tile[(E * ch + j) * PITCH + ln] = static_cast<uint8_t>(c);
      }
    }
  }
  __syncthreads();

  // ---- write: 16-byte chunk q of the tile's output, consecutive lanes along a row
  constexpr int OCPR = G::OUT_BYTES / 16;  // output chunks per row
  constexpr int OCHUNKS = G::ROWS * OCPR;
  static_assert(OCHUNKS % 256 == 0, "whole output chunks per lane");
  uint8_t* dst = p.dst + z * p.dst_batch;
#pragma unroll
  for (int i = 0; i < OCHUNKS / 256; ++i) {
    const int q = t + 256 * i;
    const int r = q / OCPR, oc = q % OCPR;
    const int64_t row = r0 + r;
    const int64_t byte = static_cast<int64_t>(blockIdx.x) * G::OUT_BYTES + 16 * oc;
    if (row >= p.rows || byte >= p.dst_ld_bytes) continue;
    uint4 o;
    if constexpr (DST == THL_E2M1X2) {
      // 32 codes, two a byte, the even element in the low nibble
      const uint4 a = *reinterpret_cast<const uint4*>(tile + r * PITCH + 32 * oc);
      const uint4 b = *reinterpret_cast<const uint4*>(tile + r * PITCH + 32 * oc + 16);
      auto nib = [](uint32_t x, uint32_t y) {  // 8 byte codes -> 8 nibbles
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) v |= ((x >> (8 * e)) & 15u) << (4 * e);
#pragma unroll
        for (int e = 0; e < 4; ++e) v |= ((y >> (8 * e)) & 15u) << (16 + 4 * e);
        return v;
      };
      o = make_uint4(nib(a.x, a.y), nib(a.z, a.w), nib(b.x, b.y), nib(b.z, b.w));
    } else {
      o = *reinterpret_cast<const uint4*>(tile + r * PITCH + 16 * oc);
    }
    *reinterpret_cast<uint4*>(dst + row * p.dst_ld_bytes + byte) = o;
  }
}

template <int SRC, int DST, bool KMAJ>
hipError_t launch_one(const CvtArgs& a, int64_t batch, hipStream_t s) {
  using G = Tile<DST, KMAJ>;
  const int64_t gx = (a.dst_ld_bytes + G::OUT_BYTES - 1) / G::OUT_BYTES;
  const int64_t gy = (a.rows + G::ROWS - 1) / G::ROWS;
  if (gx > INT32_MAX || gy > 65535 || batch > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy), static_cast<unsigned>(batch));
  hipLaunchKernelGGL((convert_kernel<SRC, DST, KMAJ>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int SRC, int DST>
hipError_t launch(const CvtArgs& a, int64_t batch, hipStream_t s) {
  return a.kmajor ? launch_one<SRC, DST, true>(a, batch, s) : launch_one<SRC, DST, false>(a, batch, s);
}

}  // namespace

hipError_t launch_convert(const CvtArgs& a, int64_t batch, hipStream_t s) {
  if (a.rows <= 0 || batch <= 0 || a.dst_ld_bytes <= 0 || a.dst_ld_bytes % 64 != 0) return hipErrorInvalidValue;
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
