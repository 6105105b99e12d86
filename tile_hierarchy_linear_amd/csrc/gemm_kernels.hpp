// gemm_kernels.hpp -- gfx950 GEMM kernels with a fused epilogue.
//
//   D = act(alpha * op(A) * op(B) + beta * C + bias[i])
//
// The tile hierarchy of the "CUTLASS" knowledge-base page ("The tile
// hierarchy"), built for CDNA4: a workgroup owns a BM x BN tile of D; its
// WM x WN wavefronts (64 lanes each) own (BM/WM) x (BN/WN) sub-tiles, each a
// grid of 32x32 MFMA tiles accumulated in registers.  K advances in steps of
// 64 bytes per operand row (32 fp16/bf16, 64 int8/fp8, 128 fp4 elements),
// so every operand format issues the same number of MFMA cycles per step.
//
// Global -> LDS (a3): buffer loads that write LDS directly (16 or 4 bytes a
// lane, no register staging) into a ring of STAGES swizzled buffers, each a
// separate LDS object so the compiler can tell a copy into one buffer from a
// read of another; copies run STAGES-1 steps ahead of the MFMAs, and their
// completion is waited for explicitly (vmcnt) before one workgroup barrier
// per step.  LDS -> registers (a4): each lane reads its MFMA fragments from
// the swizzled rows, half a step ahead of their use.  Epilogue (a7): the
// accumulators leave through LDS so that alpha/beta, bias, activation and
// conversion run on contiguous 8-row runs of D, with C read and D written
// once in whole cache lines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "gemm_args.hpp"
#include "index_maps.hpp"

namespace thl {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
// 16-byte vectors at element alignment: one access for a run of 8 elements
// whatever its offset (the HSA runtime runs the memory system in unaligned
// mode, where a vector access need only be aligned to its element size)
typedef int v4i_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef int v4i_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float v4f_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ MFMA families
// Each family: LANE_CHUNKS 16-byte chunks per lane per MFMA, KSUB MFMAs per
// 64-byte K-step, the accumulator type, and the instruction.
template <int F>
struct Fam;

template <>
struct Fam<FAM_BF16> {
  static constexpr int LANE_CHUNKS = 1, KSUB = 2;
  static constexpr bool INT = false, SCALED = false;
  using Acc = v16f;
  template <int KS>
  static __device__ __forceinline__ Acc mma(const v4i* a, const v4i* b, Acc c, int, int) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[0]), __builtin_bit_cast(v8bf, b[0]), c,
                                                   0, 0, 0);
  }
};

template <>
struct Fam<FAM_F16> {
  static constexpr int LANE_CHUNKS = 1, KSUB = 2;
  static constexpr bool INT = false, SCALED = false;
  using Acc = v16f;
  template <int KS>
  static __device__ __forceinline__ Acc mma(const v4i* a, const v4i* b, Acc c, int, int) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a[0]), __builtin_bit_cast(v8h, b[0]), c, 0,
                                                  0, 0);
  }
};

template <>
struct Fam<FAM_I8> {
  static constexpr int LANE_CHUNKS = 1, KSUB = 2;
  static constexpr bool INT = true, SCALED = false;
  using Acc = v16i;
  template <int KS>
  static __device__ __forceinline__ Acc mma(const v4i* a, const v4i* b, Acc c, int, int) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], c, 0, 0, 0);
  }
};

// The two OCP fp8 formats on one instruction: format code 0 = E4M3, 1 = E5M2,
// one code for A (FA) and one for B (FB); no block scale (constant zero scale
// operands select the unscaled instruction).
template <int FA, int FB>
struct Fam8 {
  static constexpr int LANE_CHUNKS = 2, KSUB = 1;
  static constexpr bool INT = false, SCALED = false;
  using Acc = v16f;
  template <int KS>
  static __device__ __forceinline__ Acc mma(const v4i* a, const v4i* b, Acc c, int, int) {
    const v8i av = __builtin_shufflevector(a[0], a[1], 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i bv = __builtin_shufflevector(b[0], b[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, FA, FB, 0, 0, 0, 0);
  }
};
template <>
struct Fam<FAM_FP8> : Fam8<0, 0> {};
template <>
struct Fam<FAM_E5M2> : Fam8<1, 1> {};
template <>
struct Fam<FAM_E4E5> : Fam8<0, 1> {};
template <>
struct Fam<FAM_E5E4> : Fam8<1, 0> {};

// MXFP8: fp8 elements with one E8M0 scale per 32 K-elements, format code FA
// for A and FB for B (0 = E4M3, 1 = E5M2).  The instruction applies lane l's
// scale byte to K-block l/32 of row l%32, and reads lane g's 32 bytes as K
// 16g .. 16g+15 and 32+16g .. 32+16g+15 (maps::fp8_32x32_k_of): so lane
// group g loads the step's 16-byte chunks g and g+2, and block g of the step
// is exactly the 32 stored elements its scale belongs to.
template <int FA, int FB>
struct FamMX8 {
  static constexpr int LANE_CHUNKS = 2, KSUB = 1, SPS = 2;  // SPS: scale blocks per 64-byte step
  static constexpr bool INT = false, SCALED = true;
  using Acc = v16f;
  template <int KS>
  static __device__ __forceinline__ Acc mma(const v4i* a, const v4i* b, Acc c, int sa, int sb) {
    const v8i av = __builtin_shufflevector(a[0], a[1], 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i bv = __builtin_shufflevector(b[0], b[1], 0, 1, 2, 3, 4, 5, 6, 7);
    // E8M0 scales in byte 0 of each lane's scale operand.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, FA, FB, 0, sa, 0, sb);
  }
};
template <>
struct Fam<FAM_MX8> : FamMX8<0, 0> {};
template <>
struct Fam<FAM_MX8_E5M2> : FamMX8<1, 1> {};
template <>
struct Fam<FAM_MX8_E4E5> : FamMX8<0, 1> {};
template <>
struct Fam<FAM_MX8_E5E4> : FamMX8<1, 0> {};

template <>
struct Fam<FAM_FP4> {
  static constexpr int LANE_CHUNKS = 1, KSUB = 2, SPS = 4;  // SPS: scale blocks per 64-byte step
  static constexpr bool INT = false, SCALED = true;
  using Acc = v16f;
  // Lane group g (lanes 32g .. 32g+31) takes the step's 32-element blocks 2g
  // (sub-step 0) and 2g+1 (sub-step 1); its scale register holds the two
  // E8M0 bytes of those blocks in bytes 0 and 1, and opsel picks byte KS.
  template <int KS>
  static __device__ __forceinline__ Acc mma(const v4i* a, const v4i* b, Acc c, int sa, int sb) {
    const v4i z = {0, 0, 0, 0};
    const v8i av = __builtin_shufflevector(a[0], z, 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i bv = __builtin_shufflevector(b[0], z, 0, 1, 2, 3, 4, 5, 6, 7);
    // Format 4 = E2M1 for both operands.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, KS & 1, sa, KS & 1, sb);
  }
};

// Scale blocks per 64-byte K-step of a block-scaled family (0 without scales).
template <class T>
constexpr int sps_of() {
  if constexpr (T::SCALED) return T::SPS;
  return 0;
}

// Compile-time loop: f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>).
// Guarantees unrolling where a loop body is too large for the unroller, so
// register arrays indexed by the loop variable are never demoted to memory.
template <class Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------ helpers

__device__ __forceinline__ v4i mask_bytes(v4i x, int valid) {
  // Keep the first `valid` bytes (0..16) of a 16-byte chunk, zero the rest.
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int vb = valid - 4 * w;
    const unsigned keep = vb >= 4 ? 0xffffffffu : (vb <= 0 ? 0u : ((1u << (8 * vb)) - 1u));
    x[w] = static_cast<int>(static_cast<unsigned>(x[w]) & keep);
  }
  return x;
}

__device__ __forceinline__ float load_f(const void* p, int type, int64_t i) {
  switch (type) {
    case DT_F32:
      return static_cast<const float*>(p)[i];
    case DT_F16:
      return static_cast<float>(static_cast<const _Float16*>(p)[i]);
    case DT_BF16:
      return static_cast<float>(static_cast<const __bf16*>(p)[i]);
    default:
      return 0.0f;
  }
}

__device__ __forceinline__ float activate(float t, int flags) {
  if (flags & EPI_RELU) return t > 0.0f ? t : 0.0f;
  if (flags & EPI_GELU) return 0.5f * t * (1.0f + erff(t * 0.70710678118654752440f));
  return t;
}

// Rows m .. m+rows-1 (rows <= 8) of one column of a float-family matrix, as
// floats; one or two 16-byte loads when all 8 are wanted.
__device__ __forceinline__ void load8_f(const void* base, int type, int64_t off, int rows, float (&v)[8]) {
  if (type == DT_F32) {
    const float* q = static_cast<const float*>(base) + off;
    if (rows == 8) {
      const v4f_a4 a = *reinterpret_cast<const v4f_a4*>(q), b = *reinterpret_cast<const v4f_a4*>(q + 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = a[r];
        v[4 + r] = b[r];
      }
      return;
    }
  } else {
    const uint16_t* q = static_cast<const uint16_t*>(base) + off;
    if (rows == 8) {
      const v4i_a2 w = *reinterpret_cast<const v4i_a2*>(q);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint16_t h = static_cast<uint16_t>(static_cast<unsigned>(w[r / 2]) >> (16 * (r & 1)));
        v[r] = type == DT_BF16 ? __builtin_bit_cast(float, static_cast<unsigned>(h) << 16)
                               : static_cast<float>(__builtin_bit_cast(_Float16, h));
      }
      return;
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] = r < rows ? load_f(base, type, off + r) : 0.0f;
}

// Store rows m .. m+rows-1 (rows <= 8) of one column, rounding to nearest
// even; one or two 16-byte stores when all 8 go out.
__device__ __forceinline__ void store8_f(void* base, int type, int64_t off, const float (&v)[8], int rows) {
  if (type == DT_F32) {
    float* q = static_cast<float*>(base) + off;
    if (rows == 8) {
      *reinterpret_cast<v4f_a4*>(q) = v4f_a4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<v4f_a4*>(q + 4) = v4f_a4{v[4], v[5], v[6], v[7]};
      return;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < rows) q[r] = v[r];
  } else {
    uint16_t h[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
      h[r] = type == DT_BF16 ? __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[r]))
                             : __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[r]));
    uint16_t* q = static_cast<uint16_t*>(base) + off;
    if (rows == 8) {
      *reinterpret_cast<v4i_a2*>(q) = __builtin_bit_cast(v4i, h);
      return;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < rows) q[r] = h[r];
  }
}

__device__ __forceinline__ void load8_i(const void* base, int64_t off, int rows, int (&v)[8]) {
  const int* q = static_cast<const int*>(base) + off;
  if (rows == 8) {
    const v4i_a4 a = *reinterpret_cast<const v4i_a4*>(q), b = *reinterpret_cast<const v4i_a4*>(q + 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = a[r];
      v[4 + r] = b[r];
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] = r < rows ? q[r] : 0;
}

__device__ __forceinline__ void store8_i(void* base, int64_t off, const int (&v)[8], int rows) {
  int* q = static_cast<int*>(base) + off;
  if (rows == 8) {
    *reinterpret_cast<v4i_a4*>(q) = v4i_a4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<v4i_a4*>(q + 4) = v4i_a4{v[4], v[5], v[6], v[7]};
    return;
  }
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < rows) q[r] = v[r];
}

// Buffer resource over `base` with no range limit (offsets are kept in
// bounds by the callers); raw dword data, the gfx9 default format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), -1, 0x00020000);
}

// A wave-uniform 64-bit value made visibly uniform (read from lane 0), so
// that addresses built from it stay scalar: a buffer resource the compiler
// believes divergent is issued through a loop over its distinct values.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// beta != 0 as an integer test on its bits (either zero), which stays a
// scalar value; a float compare is a vector instruction, and everything
// chosen by its result would be treated as divergent.
__device__ __forceinline__ bool nonzero_f32(float x) { return (__builtin_bit_cast(uint32_t, x) << 1) != 0; }

// Buffer resource over `num` bytes at `base`: loads at or past the end read
// zeros without touching memory, stores there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void* base, int num) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), num, 0x00020000);
}

// Buffer resource whose base and size are read from lane 0.  Built from
// values the compiler cannot prove uniform (a select on a flag is a vector
// select), a resource lands in vector registers and every load through it
// becomes a loop over the distinct values of the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_u(const void* base, int num) {
  const int64_t b = uniform64(static_cast<int64_t>(reinterpret_cast<uintptr_t>(base)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(static_cast<uintptr_t>(b)), static_cast<short>(0),
                                          __builtin_amdgcn_readfirstlane(num), 0x00020000);
}

// 16-byte buffer load at the resource base + voffset + soffset.
__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t vo, int so) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0));
}
// 16-byte buffer store at the resource base + voffset + so, with the whole
// offset in the vector operand and a zero soffset.  A store of more than 8
// bytes reads its data registers over the cycles after it issues, so a VALU
// write of those registers must wait a few cycles.  The compiler inserts
// that wait for buffer stores with a zero soffset (and for global stores),
// but not for ones whose soffset is a scalar register: there, a register
// reused at once for the next run's arithmetic was stored instead of the
// packed outputs (first dword of some lanes' 16-byte runs).
__device__ __forceinline__ void buf_store16(v4i v, __amdgpu_buffer_rsrc_t r, uint32_t vo, int so) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, vo + static_cast<uint32_t>(so), 0, 0);
}

// ------------------------------------------------------------ MX output
// One block of an MX output: the OCP MX rule applied to the fp32 epilogue
// values (shared exponent floor(log2 amax) - emax, clamped to E8M0's range;
// elements rounded to nearest even, larger magnitudes clamped to the largest
// finite element, signs kept).

// floor(log2(x)) of a finite x > 0 from its bits (subnormals included).
__device__ __forceinline__ int floor_log2_f32(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x) & 0x7fffffffu;
  const int e = static_cast<int>(b >> 23);
  if (e != 0) return e - 127;
  return -149 + (31 - __builtin_clz(b));  // subnormal: the top set mantissa bit
}

// E8M0 code of the block whose largest magnitude is amax (>= 0), for an
// element format whose largest exponent is emax; 0 for a block of zeros.
__device__ __forceinline__ int mx_scale_code(float amax, int emax) {
  if (!(amax > 0.0f)) return 0;
  int x = floor_log2_f32(amax) - emax;
  x = x < -127 ? -127 : (x > 127 ? 127 : x);
  return x + 127;
}

// E2M1 code of v (already divided by the block scale): the nearest of
// 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even code, above 6 clamped to 6.
__device__ __forceinline__ unsigned e2m1_code(float v) {
  const float a = __builtin_fabsf(v);
  unsigned c = 0;
  c += (a > 0.25f) ? 1u : 0u;
  c += (a >= 0.75f) ? 1u : 0u;  // tie at 0.75 goes up to the even code 2
  c += (a > 1.25f) ? 1u : 0u;
  c += (a >= 1.75f) ? 1u : 0u;  // tie at 1.75 -> code 4
  c += (a > 2.5f) ? 1u : 0u;
  c += (a >= 3.5f) ? 1u : 0u;   // tie at 3.5 -> code 6
  c += (a > 5.0f) ? 1u : 0u;
  return c | ((__builtin_bit_cast(uint32_t, v) >> 28) & 8u);
}

// Bitwise select (a where m is set, else b): keeps a uniform type or flag
// choice a per-lane select instead of a branch around each element.
__device__ __forceinline__ unsigned bsel(unsigned m, unsigned a, unsigned b) { return (a & m) | (b & ~m); }

// Eight packed 16-bit values as floats; `bf` is all ones for bf16, zero for
// f16.
__device__ __forceinline__ void unpack8(const v4i w, unsigned bf, float (&v)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const unsigned u = static_cast<unsigned>(w[r / 2]);
    const unsigned hb = __builtin_bit_cast(
        unsigned, static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> (16 * (r & 1))))));
    v[r] = __builtin_bit_cast(float, bsel(bf, (r & 1) ? (u & 0xffff0000u) : (u << 16), hb));
  }
}

// Eight floats packed to bf16 or f16 (as for unpack8), rounded to nearest even.
__device__ __forceinline__ v4i pack8(const float (&v)[8], unsigned bf) {
  v4i w;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const unsigned b = static_cast<unsigned>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * q]))) |
                       (static_cast<unsigned>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * q + 1]))) << 16);
    const unsigned h = static_cast<unsigned>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v[2 * q]))) |
                       (static_cast<unsigned>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(v[2 * q + 1]))) << 16);
    w[q] = static_cast<int>(bsel(bf, b, h));
  }
  return w;
}

// Direct buffer -> LDS load of W bytes per lane at base + voffset.
template <int W>
__device__ __forceinline__ void load_lds_buf(__amdgpu_buffer_rsrc_t r, uint32_t voffset, void* lds) {
  auto* l = (__attribute__((address_space(3))) void*)(lds);
  if constexpr (W == 16) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voffset, 0, 0, 0);
  } else {
    static_assert(W == 4, "16- or 4-byte lanes");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 4, voffset, 0, 0, 0);
  }
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt low bits [3:0], high bits [15:14]; expcnt and
// lgkmcnt left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence __syncthreads() adds (that
// fence waits for every outstanding vector-memory operation, including the
// copies of later stages).  The empty asm statements keep the compiler from
// moving LDS accesses across it; data waits are explicit.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One LDS buffer of the staging ring per (size, index): separate objects, so
// the compiler can tell a copy into one slot from a read of another and does
// not make the read wait for the copy.
template <int BYTES, int I>
__device__ __forceinline__ uint8_t* ring_slot() {
  __shared__ __attribute__((aligned(1024))) uint8_t slot[BYTES];
  return slot;
}


// The two fp4 scale-group buffers (separate objects, like the ring slots).
template <int BYTES, int I>
__device__ __forceinline__ uint8_t* scale_group() {
  __shared__ __attribute__((aligned(16))) uint8_t buf[BYTES];
  return buf;
}

// The epilogue's own LDS staging area (separate from the ring).
template <int BYTES>
__device__ __forceinline__ uint8_t* ep_area() {
  __shared__ __attribute__((aligned(1024))) uint8_t area[BYTES];
  return area;
}

// Batched problems (L mode, the "CUTLASS" knowledge-base page's batched
// GEMM): problem z's operands, scales, C, bias and D sit at fixed byte
// strides from the first problem's.
__device__ __forceinline__ void offset_to_problem(GemmArgs& p, const int64_t z) {
  p.a += z * p.bs_a;
  p.b += z * p.bs_b;
  p.sfa += z * p.bs_sfa;
  p.sfb += z * p.bs_sfb;
  p.c = static_cast<const uint8_t*>(p.c) + z * p.bs_c;
  p.d = static_cast<uint8_t*>(p.d) + z * p.bs_d;
  p.bias = static_cast<const uint8_t*>(p.bias) + z * p.bs_bias;
}

// Grouped problems (the grouped GEMM of "What's New in CUTLASS 4.8"): grid
// column blockIdx.x computes problem group[blockIdx.x], whose sizes, pointers
// and leading dimensions replace the launch-wide ones.  Returns false when
// this workgroup has no tile of that problem (the whole workgroup leaves).
template <int BM, int BN>
__device__ __forceinline__ bool select_group_problem(GemmArgs& p) {
  const GroupProblem& g = p.group[blockIdx.x];
  const int64_t m = g.m, n = g.n, k = g.k;
  p.m = static_cast<int32_t>(m);
  p.n = static_cast<int32_t>(n);
  p.k = static_cast<int32_t>(k);
  p.kbytes = static_cast<int32_t>(k * p.elem_bits_a / 8);
  p.a = static_cast<const uint8_t*>(g.a);
  p.b = static_cast<const uint8_t*>(g.b);
  p.c = g.c;
  p.d = g.d;
  p.bias = (p.flags & EPI_BIAS) ? g.bias : nullptr;
  p.sfa = g.sfa;
  p.sfb = g.sfb;
  p.lda_bytes = g.lda * p.elem_bits_a / 8;
  p.ldb_bytes = g.ldb * p.elem_bits_b / 8;
  p.ldc = g.ldc;
  p.ldd = g.ldd;
  p.ld_sfa = g.ld_sfa;
  p.ld_sfb = g.ld_sfb;
  p.tiles_m = static_cast<int32_t>((m + BM - 1) / BM);
  p.tiles_n = static_cast<int32_t>((n + BN - 1) / BN);
  return m > 0 && n > 0 && static_cast<int64_t>(blockIdx.y) < static_cast<int64_t>(p.tiles_m) * p.tiles_n;
}

// ------------------------------------------------------------ the kernel
//
// Pipeline (per wavefront, K-steps of 64 bytes per operand row, a ring of
// STAGES LDS buffers, copies always issued STAGES-1 steps ahead):
//
//   step kt, phase A:  first half of step kt's MFMAs; LDS reads of the
//                      fragments for the second half (from buffer kt).
//   barrier:           after this wave's copies of stage kt+1 have landed
//                      (those of later stages may still be in flight); past
//                      it, stage kt+1 is visible and every wave has finished
//                      step kt-1, so buffer kt-1 is free.
//   step kt, phase B:  second half of step kt's MFMAs; copies of stage
//                      kt+STAGES-1 into the freed buffer; LDS reads of step
//                      kt+1's first fragments (and fp4 scales).
//
// Each phase is a scheduling region of its own (nothing crosses the
// barrier), inside which the reads are spread over the MFMAs and finish two
// MFMAs before the phase ends.  The copies past the last full step re-read
// the last full step (uniform, in bounds) so every step issues the same
// number of copies; a partial final K-step is loaded and computed after the
// loop with bytes past K masked to zero.
//
// Operand storage: AK (BK) true when op(A) rows (op(B) columns) are
// contiguous along K (opA = T, opB = N), staged as rows of 64 bytes of K;
// false when they are contiguous along M (N) -- 16-bit types only -- staged
// as 32 k-rows of the tile's M (N) extent and turned into K-contiguous
// fragments by two transposed 16-bit LDS reads each.
//
// MXO: the variant writes MX-format D (elements plus generated E8M0 scales,
// GemmArgs::mx_out); built as variants of their own so that no other kernel
// carries its code.
template <int F, int BM, int BN, int WM, int WN, int LOADW, int STAGES, int OCC, int SCW, bool AK, bool BK,
          bool MXO = false>
__global__ void __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
gemm_kernel(GemmArgs p) {
  // Grid: problem blockIdx.x (one for a single problem), persistent
  // workgroup blockIdx.y of gridDim.y per problem.
  if (p.group) {
    if (!select_group_problem<BM, BN>(p)) return;
  } else {
    offset_to_problem(p, blockIdx.x);
  }
  using T = Fam<F>;
  using Acc = typename T::Acc;
  constexpr int KB = maps::kStepBytes;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int LC = T::LANE_CHUNKS, KSUB = T::KSUB, CPM = (KB / 16) / KSUB;
  constexpr int A_BYTES = BM * KB, B_BYTES = BN * KB;
  constexpr int A_LOADS = A_BYTES / (64 * LOADW * NW), B_LOADS = B_BYTES / (64 * LOADW * NW);
  constexpr int COPIES = A_LOADS + B_LOADS;  // operand copies per wave per stage
  constexpr int NSC = T::SCALED ? FM + FN : 1;
  // fp4 block scales travel in groups of SG = 4 K-steps: one 16-byte lane
  // per A and B row brings the group's 16 E8M0 bytes (scale rows must be
  // 16-byte aligned), into one of two group buffers that alternate.  The
  // copies of group g go out with stage 4g; the per-wave count is padded to
  // a whole number with copies into a dummy area so every wave issues the
  // same.  (One 4-byte lane per row per step touched as many cache lines as
  // all the operand copies of the step.)
  static_assert(SCW == 16, "scale copies bring 16 bytes (16 blocks) a row");
  static_assert(BM % 64 == 0, "a scale copy instruction covers 64 rows of one operand");
  // K-steps per scale group: 4 for fp4 (4 blocks a step), 8 for MXFP8 (2)
  constexpr int SG = T::SCALED ? SCW / sps_of<T>() : 4;
  constexpr int SC_BYTES = T::SCALED ? (BM + BN) * SCW : 0;  // one group buffer
  constexpr int SC_INSTR = T::SCALED ? (BM + BN) / 64 : 0;
  constexpr int SC_LOADS = T::SCALED ? (SC_INSTR + NW - 1) / NW : 0;
  constexpr int SC_PAD = (T::SCALED && SC_INSTR % NW != 0) ? 64 * SCW : 0;
  constexpr int SC_BUF = SC_BYTES + SC_PAD;  // one group buffer (with the dummy area)
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int VM_STAGE = COPIES;  // operand copies per wave per stage
  // Copies per wave of the stage at position pos (a multiple of SG carries
  // its scale group too).
  auto vm_of = [](int pos) constexpr { return COPIES + (pos % SG == 0 ? SC_LOADS : 0); };
  static_assert(STAGE % 16 == 0, "stages stay 16-byte aligned");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole MFMA tiles");
  static_assert(A_LOADS * 64 * LOADW * NW == A_BYTES && B_LOADS * 64 * LOADW * NW == B_BYTES,
                "copies must split evenly over waves");
  static_assert(STAGES >= 3 && STAGES <= 6, "three to six stages");
  static_assert((VM_STAGE + SC_LOADS) * (STAGES - 2) < 64, "vmcnt range");
  // Paired stages (four buffers, 16-byte copies): stages 2j and 2j+1 share a
  // buffer pair and go out together, in the step before 2j-1, so that every
  // copy of a K-major operand reads whole 128-byte lines (maps::pair_*).  The
  // pair's buffers are free once stage 2j-1 has been read, and stage 2j is
  // first read two steps later, as with single stages.
  constexpr bool PAIR = STAGES == 4 && LOADW == 16;
  static_assert(!PAIR || NW % 4 == 0, "a wave's pair copies keep one chunk swizzle");
  constexpr int RSTEP = PAIR ? 2 * KB : KB;  // LDS bytes per K-major row of an 8-row group
  // Phase A MFMAs: all of sub-step 0 (two sub-steps per K-step), else the
  // first half of the rows (measured 2% faster for e4m3 than a quarter).
  constexpr int RA = KSUB == 2 ? FM : FM / 2;
  // Steps per unrolled loop body: ring slots, fragment-slot parities and (fp4)
  // the scale-group buffer and position are compile-time constants inside it.
  constexpr int UNROLL = T::SCALED ? (STAGES % (2 * SG) == 0 ? STAGES : ((2 * SG) % STAGES == 0 ? 2 * SG : 0))
                                   : ((STAGES % 2 == 0) ? STAGES : 2 * STAGES);
  static_assert(UNROLL > 0, "scale groups need STAGES to divide into 4 K-step groups");
  // Copies per wave issued in phase B of the step at position pos: paired,
  // odd steps issue stages pos+3 and pos+4 (with the scale group that starts
  // at pos+5, when one does), even steps none; otherwise every step issues
  // stage pos+3.
  auto issued_at = [](int pos) constexpr {
    if constexpr (PAIR) return (pos % 2 != 0) ? 2 * COPIES + ((pos + 5) % SG == 0 ? SC_LOADS : 0) : 0;
    return COPIES + ((pos + STAGES - 1) % SG == 0 ? SC_LOADS : 0);
  };
  // Copies per wave younger than stage pos+1 when waiting for it at step pos
  // (single: stages pos+2 .. pos+STAGES-2 may still be in flight; paired:
  // the pair issued at step pos-1 when stage pos+1 is odd).
  auto younger = [](int pos) constexpr {
    if constexpr (PAIR) return (pos % 2 == 0) ? 2 * COPIES + ((pos + 4) % SG == 0 ? SC_LOADS : 0) : 0;
    int n = 0;
    for (int q = pos + 2; q <= pos + STAGES - 2; ++q) n += COPIES + (q % SG == 0 ? SC_LOADS : 0);
    return n;
  };
  static_assert(KSUB == 2 || (KSUB == 1 && FM % 2 == 0), "a step splits into two halves");
  static_assert((AK && BK) || F == FAM_BF16 || F == FAM_F16, "M/N-major operands are 16-bit only");
  constexpr int PA = BM * 2, PB = BN * 2;  // k-row pitch of M- (N-) major stages
  static_assert(AK || PA % 256 == 0, "M-major k-rows are whole 256-byte bank windows");
  static_assert(BK || PB % 256 == 0, "N-major k-rows are whole 256-byte bank windows");

  // Paired: two buffer pairs of 2*STAGE bytes (A's two stages, then B's);
  // slot(i) is then the i-th STAGE bytes of the ring, for raw staging only.
  auto pair_buf = [](auto j_tag) -> uint8_t* { return ring_slot<2 * STAGE, decltype(j_tag)::value>(); };
  auto slot = [&](auto i_tag) -> uint8_t* {
    constexpr int I = decltype(i_tag)::value;
    if constexpr (PAIR) {
      return pair_buf(std::integral_constant<int, I / 2>{}) + (I % 2) * STAGE;
    } else {
      return ring_slot<STAGE, I>();
    }
  };
  // Operand bases of the stage held in buffer I: K-major stages of a pair
  // interleave by 8-row groups (the odd one 512 bytes in), M-major ones
  // follow each other.
  auto a_stage = [&](auto i_tag) -> uint8_t* {
    constexpr int I = decltype(i_tag)::value;
    if constexpr (PAIR) {
      return pair_buf(std::integral_constant<int, I / 2>{}) + (I % 2) * (AK ? 512 : A_BYTES);
    } else {
      return slot(i_tag);
    }
  };
  auto b_stage = [&](auto i_tag) -> uint8_t* {
    constexpr int I = decltype(i_tag)::value;
    if constexpr (PAIR) {
      return pair_buf(std::integral_constant<int, I / 2>{}) + 2 * A_BYTES + (I % 2) * (BK ? 512 : B_BYTES);
    } else {
      return slot(i_tag) + A_BYTES;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int ntiles = p.tiles_m * p.tiles_n;
  // Split K: work unit u is split u % splits of tile u / splits and covers
  // p.ksteps K-steps from the split's first (the last split keeps the
  // partial step); without it, one unit per tile.  nk, nkf, kbytes_u and
  // kel_u describe the current unit's K range.  Each split writes its
  // partial product, unscaled, to a matrix of its own: D here is the first
  // of `splits` fp32 (int32) matrices p.split_stride bytes apart, which a
  // second kernel adds in split order before the epilogue proper.
  // Split K is built into the 128x128 two-workgroup variants of the unscaled
  // families (the tiles chosen when a problem has few); elsewhere splits is 1.
  constexpr bool SPLITK = OCC == 2 && BM * BN <= 128 * 128 && !T::SCALED;
  const int splits = (SPLITK && p.splits > 1) ? p.splits : 1;
  const int nk_all = (p.kbytes + KB - 1) / KB;
  const int nunits = ntiles * splits;
  int nk = nk_all;         // K-steps of the unit, the last one possibly partial
  int nkf = p.kbytes / KB; // full K-steps of the unit
  int kbytes_u = p.kbytes; // bytes of K per operand row in the unit
  int kel_u = p.k;         // elements of K in the unit
  int unit_tile = 0, unit_split = 0;
  void* d_unit = p.d;  // the current unit's output matrix
  const int64_t a_step = AK ? KB : 32 * p.lda_bytes;  // operand advance per K-step
  const int64_t b_step = BK ? KB : 32 * p.ldb_bytes;
  const int nkb = p.k >> 5;
  const __amdgpu_buffer_rsrc_t rs_sfa = make_rsrc(p.sfa), rs_sfb = make_rsrc(p.sfb);

  // Per-tile state: the tile's origin, operand bases (uniform) and the
  // per-lane 32-bit byte offsets of every copy this wave issues.  K-major:
  // rows past M (N) re-read the last valid row.  M-major: 16-byte chunks
  // wholly past M (N) re-read the tile's first chunk of that k-row.  fp4:
  // the source row of each scale copy.
  int64_t m0 = 0, n0 = 0;
  const uint8_t* a_tile = p.a;
  const uint8_t* b_tile = p.b;
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
  // Paired K-major copies: the lane's offset for instruction 0 (rows of the
  // wave's first 8-row group); instruction j is 8*NW*j rows further.  Rows
  // past M (N) are cut off by the buffer resource's size instead of clamped.
  uint32_t a_lp = 0, b_lp = 0;
  uint32_t sc_src[T::SCALED ? SC_LOADS : 1];
  bool sc_a[T::SCALED ? SC_LOADS : 1];
  int sc_dst[T::SCALED ? SC_LOADS : 1];
  // Workgroups visit tiles id = blockIdx.y, + gridDim.y, ...; the XCD remap
  // and grouped raster turn id into (tm, tn) so that the tiles one XCD works
  // on at a time share A and B panels in its L2 (gridDim.y is a multiple of
  // 8 whenever the tile count is).  The hardware deals workgroups to the 8
  // XCDs by their linear id x + y * gridDim.x: with a multiple of 8
  // problems every workgroup of a problem runs on one XCD (p.xcd_local), and
  // the raster alone keeps its concurrent tiles together.
  auto setup = [&](int id) {
    int64_t tm, tn;
    if (SPLITK && splits > 1) {
      // the splits of one tile are consecutive units (consecutive workgroups)
      unit_tile = id / splits;
      unit_split = id - unit_tile * splits;
      maps::grouped_tile(unit_tile, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    } else {
      maps::grouped_tile(p.xcd_local ? id : maps::xcd_remap(id, ntiles), p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    }
    m0 = tm * BM;
    n0 = tn * BN;
    a_tile = AK ? p.a + m0 * p.lda_bytes : p.a + m0 * 2;
    b_tile = BK ? p.b + n0 * p.ldb_bytes : p.b + n0 * 2;
    if (SPLITK && splits > 1) {
      const int kbeg = unit_split * p.ksteps;
      const int kend = kbeg + p.ksteps < nk_all ? kbeg + p.ksteps : nk_all;
      const int bend = kend * KB < p.kbytes ? kend * KB : p.kbytes;
      kbytes_u = bend - kbeg * KB;
      kel_u = p.k - kbeg * (KB / 2);  // M-major operands are 16-bit: 32 elements a step
      nk = kend - kbeg;
      nkf = kbytes_u / KB;
      a_tile += kbeg * a_step;
      b_tile += kbeg * b_step;
      d_unit = static_cast<uint8_t*>(p.d) + unit_split * p.split_stride;
    }
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
      int64_t row, byte;
      if constexpr (AK) {
        maps::copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, &row, &byte);
        const int64_t r = (m0 + row < p.m ? m0 + row : p.m - 1) - m0;
        a_off[j] = static_cast<uint32_t>(r * p.lda_bytes + byte);
      } else {
        maps::mm_copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, PA, &row, &byte);
        if (m0 + (byte & ~15) / 2 >= p.m) byte &= 15;
        a_off[j] = static_cast<uint32_t>(row * p.lda_bytes + byte);
      }
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
      int64_t row, byte;
      if constexpr (BK) {
        maps::copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, &row, &byte);
        const int64_t r = (n0 + row < p.n ? n0 + row : p.n - 1) - n0;
        b_off[j] = static_cast<uint32_t>(r * p.ldb_bytes + byte);
      } else {
        maps::mm_copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, PB, &row, &byte);
        if (n0 + (byte & ~15) / 2 >= p.n) byte &= 15;
        b_off[j] = static_cast<uint32_t>(row * p.ldb_bytes + byte);
      }
    }
    if constexpr (PAIR) {
      int64_t row, byte;
      maps::pair_copy_source(wave, lane, &row, &byte);
      if constexpr (AK) a_lp = static_cast<uint32_t>(row * p.lda_bytes + byte);
      if constexpr (BK) b_lp = static_cast<uint32_t>(row * p.ldb_bytes + byte);
    }
    if constexpr (T::SCALED) {
#pragma unroll
      for (int t = 0; t < SC_LOADS; ++t) {
        // One copy instruction covers 64 rows, all of A or all of B (BM is a
        // multiple of 64), so the choice is uniform over the wave and the
        // buffer resource stays scalar.
        const int j = t * NW + wave;
        const int row0 = j < SC_INSTR ? j * 64 : 0;
        sc_a[t] = row0 < BM;
        if (sc_a[t]) {
          const int64_t r = m0 + row0 + lane < p.m ? m0 + row0 + lane : p.m - 1;
          sc_src[t] = static_cast<uint32_t>(r * p.ld_sfa);  // row base; + 16 bytes per group
        } else {
          const int64_t r = n0 + (row0 - BM) + lane < p.n ? n0 + (row0 - BM) + lane : p.n - 1;
          sc_src[t] = static_cast<uint32_t>(r * p.ld_sfb);
        }
        sc_dst[t] = j < SC_INSTR ? j * 64 * SCW : SC_BYTES;
      }
    }
  };

  // The scale group buffers (fp4).
  auto sgbuf = [](auto i_tag) -> uint8_t* { return scale_group<SC_BUF, decltype(i_tag)::value>(); };
  // The scale copies of group g into group buffer GB: row bytes 16g .. 16g+15;
  // a group at or past the rows' last block re-reads the row's first group
  // (never used).
  auto issue_scale = [&](int t, int g, uint8_t* buf) {
    const int o = 16 * g;
    load_lds_buf<SCW>(sc_a[t] ? rs_sfa : rs_sfb, sc_src[t] + (o < nkb ? o : 0), buf + sc_dst[t]);
  };
  // Copy V of the stage at position POS (kt is its K-step) into ring slot
  // BUF: the scale copies first when POS starts a group, then A's, then B's;
  // ra / rb are the step's operand bases.
  auto issue_one = [&](auto v_tag, auto buf_tag, auto pos_tag, int kt, __amdgpu_buffer_rsrc_t ra,
                       __amdgpu_buffer_rsrc_t rb) {
    constexpr int V = decltype(v_tag)::value, BUF = decltype(buf_tag)::value, POS = decltype(pos_tag)::value;
    constexpr int NS = vm_of(POS) - COPIES;  // scale copies of this stage
    uint8_t* sa = slot(std::integral_constant<int, BUF>{});
    if constexpr (V < NS) {
      issue_scale(V, kt / SG, sgbuf(std::integral_constant<int, (POS / SG) % 2>{}));
    } else if constexpr (V < NS + A_LOADS) {
      constexpr int J = V - NS;
      load_lds_buf<LOADW>(ra, a_off[J], sa + (J * NW + wave) * 64 * LOADW);
    } else {
      constexpr int J = V - NS - A_LOADS;
      load_lds_buf<LOADW>(rb, b_off[J], sa + A_BYTES + (J * NW + wave) * 64 * LOADW);
    }
  };
  auto step_src = [&](int kt, __amdgpu_buffer_rsrc_t& ra, __amdgpu_buffer_rsrc_t& rb) {
    ra = make_rsrc(a_tile + kt * a_step);
    rb = make_rsrc(b_tile + kt * b_step);
  };
  // Every copy of the stage at position POS (K-step kt) into ring slot BUF.
  auto issue_full = [&](int kt, auto buf_tag, auto pos_tag) {
    __amdgpu_buffer_rsrc_t ra, rb;
    step_src(kt, ra, rb);
    static_for<vm_of(decltype(pos_tag)::value)>([&](auto vc) { issue_one(vc, buf_tag, pos_tag, kt, ra, rb); });
  };

  // Paired copies.  The K-major sources of the pair whose first stage is s0:
  // a resource from the pair's first byte of the tile, sized to end at the
  // operand's last valid byte (rows past M read zeros).
  auto pair_src = [&](int s0, __amdgpu_buffer_rsrc_t& ra, __amdgpu_buffer_rsrc_t& rb) {
    const int64_t kb = static_cast<int64_t>(s0) * KB;
    if constexpr (AK) {
      int64_t na = (p.m - 1 - m0) * p.lda_bytes + kbytes_u - kb;
      na = na < BM * p.lda_bytes ? na : BM * p.lda_bytes;
      ra = make_rsrc_n(a_tile + kb, static_cast<int>(na > 0 ? na : 0));
    } else {
      ra = make_rsrc(a_tile);
    }
    if constexpr (BK) {
      int64_t nb = (p.n - 1 - n0) * p.ldb_bytes + kbytes_u - kb;
      nb = nb < BN * p.ldb_bytes ? nb : BN * p.ldb_bytes;
      rb = make_rsrc_n(b_tile + kb, static_cast<int>(nb > 0 ? nb : 0));
    } else {
      rb = make_rsrc(b_tile);
    }
  };
  // Copies per wave of the pair whose first stage sits at position pos.  A
  // pair carries the scale group that starts two stages after it (fp4): the
  // group of steps 4g+8 .. 4g+11 goes out after step 4g+3's barrier, into the
  // buffer of group g+0 (last read in phase A of step 4g+2), and has landed
  // by step 4g+5's barrier, so that every step reads the next step's scales
  // in its phase A, with no scale read after a barrier.
  auto pair_count = [](int pos) constexpr { return 2 * COPIES + ((pos + 2) % SG == 0 ? SC_LOADS : 0); };
  // A pair's copies go out over the MFMAs of phase B of the odd step before
  // it and phase A of the next (even) step, in proportion to their MFMAs:
  // the first pair_first(pos) in phase B, the rest in phase A.
  constexpr int NMA = RA * FN;
  constexpr int NMB = (KSUB == 2 ? FM : FM - RA) * FN;
  auto pair_first = [](int pos) constexpr {
    return (2 * COPIES + ((pos + 2) % SG == 0 ? SC_LOADS : 0)) * NMB / (NMA + NMB);
  };
  // Copy V of the pair (stage s0 at position POS, s0+1) into buffer pair BUF:
  // the scale copies first when POS+2 starts a group, then A's, then B's.  A
  // pair clamped at the last K-step carries a group that no step uses.
  // K-major: one 1 KB group of 8 rows x 128 bytes per instruction; M-major:
  // each stage's copies as for single stages (k-rows of whole lines already).
  auto issue_pair_one = [&](auto v_tag, auto buf_tag, auto pos_tag, int s0, __amdgpu_buffer_rsrc_t ra,
                            __amdgpu_buffer_rsrc_t rb) {
    constexpr int V = decltype(v_tag)::value, BUF = decltype(buf_tag)::value, POS = decltype(pos_tag)::value;
    constexpr int NS = pair_count(POS) - 2 * COPIES;
    uint8_t* pa = pair_buf(std::integral_constant<int, BUF>{});
    uint8_t* pb = pa + 2 * A_BYTES;
    if constexpr (V < NS) {
      issue_scale(V, (s0 + 2) / SG, sgbuf(std::integral_constant<int, ((POS + 2) / SG) % 2>{}));
    } else if constexpr (V < NS + 2 * A_LOADS) {
      constexpr int J = V - NS;
      if constexpr (AK) {
        load_lds_buf<16>(ra, a_lp + static_cast<uint32_t>(J * 8 * NW) * static_cast<uint32_t>(p.lda_bytes),
                         pa + (J * NW + wave) * 1024);
      } else {
        constexpr int H = J / A_LOADS, JJ = J % A_LOADS;
        const int s = s0 + H < nkf ? s0 + H : nkf - 1;
        load_lds_buf<LOADW>(make_rsrc(a_tile + s * a_step), a_off[JJ], pa + H * A_BYTES + (JJ * NW + wave) * 64 * LOADW);
      }
    } else {
      constexpr int J = V - NS - 2 * A_LOADS;
      if constexpr (BK) {
        load_lds_buf<16>(rb, b_lp + static_cast<uint32_t>(J * 8 * NW) * static_cast<uint32_t>(p.ldb_bytes),
                         pb + (J * NW + wave) * 1024);
      } else {
        constexpr int H = J / B_LOADS, JJ = J % B_LOADS;
        const int s = s0 + H < nkf ? s0 + H : nkf - 1;
        load_lds_buf<LOADW>(make_rsrc(b_tile + s * b_step), b_off[JJ], pb + H * B_BYTES + (JJ * NW + wave) * 64 * LOADW);
      }
    }
  };
  // Every copy of the pair whose first stage is s0 (position POS) into BUF.
  auto issue_pair_full = [&](int s0, auto buf_tag, auto pos_tag) {
    __amdgpu_buffer_rsrc_t ra, rb;
    pair_src(s0, ra, rb);
    static_for<pair_count(decltype(pos_tag)::value)>([&](auto vc) { issue_pair_one(vc, buf_tag, pos_tag, s0, ra, rb); });
  };

  // The partial last K-step into slot 0: K-major bytes at or past K read the
  // row's first byte instead, M-major k-rows at or past K read the step's
  // first k-row (masked before the MFMAs).
  auto issue_partial = [&](int kt) {
    uint8_t* sa = a_stage(I0{});
    uint8_t* sb = b_stage(I0{});
    const int64_t kofs = static_cast<int64_t>(kt) * KB;
    if constexpr (T::SCALED) {
      uint8_t* gb = ((kt / SG) & 1) ? sgbuf(I1{}) : sgbuf(I0{});
#pragma unroll
      for (int t = 0; t < SC_LOADS; ++t) issue_scale(t, kt / SG, gb);
    }
    // K-major: offsets from the tile base; M-major: from the step's first k-row.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(AK ? a_tile : a_tile + kt * a_step);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(BK ? b_tile : b_tile + kt * b_step);
    if constexpr (PAIR && AK) {
      // paired layout: 8-row groups of 128 bytes (the odd half unused)
#pragma unroll
      for (int j = 0; j < 2 * A_LOADS; ++j) {
        int64_t row, byte;
        maps::pair_copy_source(j * NW + wave, lane, &row, &byte);
        const int64_t r = m0 + row < p.m ? row : p.m - 1 - m0;
        const int64_t off = r * p.lda_bytes + (kofs + byte < kbytes_u ? kofs + byte : 0);
        load_lds_buf<16>(ra, static_cast<uint32_t>(off), sa + (j * NW + wave) * 1024);
      }
    }
#pragma unroll
    for (int j = 0; j < ((PAIR && AK) ? 0 : A_LOADS); ++j) {
      int64_t row, byte, off;
      if constexpr (AK) {
        maps::copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, &row, &byte);
        off = a_off[j] + (kofs + byte < kbytes_u ? kofs : -byte);
      } else {
        maps::mm_copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, PA, &row, &byte);
        const int64_t k = 32 * static_cast<int64_t>(kt) + row;
        off = a_off[j] - (k < kel_u ? 0 : row * p.lda_bytes);
      }
      load_lds_buf<LOADW>(ra, static_cast<uint32_t>(off), sa + (j * NW + wave) * 64 * LOADW);
    }
    if constexpr (PAIR && BK) {
#pragma unroll
      for (int j = 0; j < 2 * B_LOADS; ++j) {
        int64_t row, byte;
        maps::pair_copy_source(j * NW + wave, lane, &row, &byte);
        const int64_t r = n0 + row < p.n ? row : p.n - 1 - n0;
        const int64_t off = r * p.ldb_bytes + (kofs + byte < kbytes_u ? kofs + byte : 0);
        load_lds_buf<16>(rb, static_cast<uint32_t>(off), sb + (j * NW + wave) * 1024);
      }
    }
#pragma unroll
    for (int j = 0; j < ((PAIR && BK) ? 0 : B_LOADS); ++j) {
      int64_t row, byte, off;
      if constexpr (BK) {
        maps::copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, &row, &byte);
        off = b_off[j] + (kofs + byte < kbytes_u ? kofs : -byte);
      } else {
        maps::mm_copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, PB, &row, &byte);
        const int64_t k = 32 * static_cast<int64_t>(kt) + row;
        off = b_off[j] - (k < kel_u ? 0 : row * p.ldb_bytes);
      }
      load_lds_buf<LOADW>(rb, static_cast<uint32_t>(off), sb + (j * NW + wave) * 64 * LOADW);
    }
  };

  Acc acc[FM][FN];

  // Per-lane LDS offset of the chunk read for MFMA sub-step ks: fragment rows
  // differ by multiples of 32, which leave the swizzle unchanged, so one
  // offset per sub-step serves every fragment row (plus a constant).
  const int lrow = lane & 31;
  // The 16-byte chunk of the step's 64 bytes that lane group g (lanes 32g ..)
  // reads as chunk c of sub-step ks.  A and B use the same assignment, so any
  // order of K within a step cancels in the dot product; fp4 gives each group
  // two adjacent 32-element blocks so that its scale bytes are adjacent too.
  auto chunk_of = [](int ks, int g, int c) {
    if constexpr (T::SCALED && LC == 2) return g + 2 * c;  // MXFP8: one scale block per lane group
    return T::SCALED ? g * KSUB + ks : ks * CPM + g * LC + c;
  };
  int chunk_off[KSUB][LC];
#pragma unroll
  for (int ks = 0; ks < KSUB; ++ks)
#pragma unroll
    for (int c = 0; c < LC; ++c)
      chunk_off[ks][c] = static_cast<int>(maps::lds_offset(lrow, chunk_of(ks, lane >> 5, c) * 16)) +
                         (PAIR ? (lrow >> 3) * 512 : 0);
  // K-major fragment rows start at multiples of 32, where a row's offset is
  // RSTEP bytes per row (paired stages interleave by 8-row groups).
  const int a_wave_off = wm * TM * RSTEP, b_wave_off = wn * TN * RSTEP;

  v4i af[2][FM][LC], bf[2][FN][LC];  // fragment slots: (kt*KSUB + ks) & 1

  // M/N-major fragments: lane addresses for the two transposed reads of
  // sub-step ks (k within the step and the row within a 32-row fragment).
  int tr_k[KSUB][2], tr_m[2];
#pragma unroll
  for (int ks = 0; ks < KSUB; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int64_t k, m;
      maps::tr16_operand(lane, h, &k, &m);
      tr_k[ks][h] = static_cast<int>(k) + ks * 16;
      tr_m[h] = static_cast<int>(m);
    }

  // Read one M-major 16-bit fragment (rows r0 .. r0+31 of the stage's
  // operand, k-range of sub-step KS) and zero the values at or past k = kv.
  auto read_mm = [&](const uint8_t* base, int pitch, int r0, auto ks_tag, int kv) -> v4i {
    constexpr int KS = decltype(ks_tag)::value;
    v2i half[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = tr_k[KS][h];
      const int off = static_cast<int>(maps::mm_lds_offset(k, 2 * (r0 + tr_m[h]), pitch));
      typedef short v4s __attribute__((ext_vector_type(4)));
      const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(base + off));
      v2i w = __builtin_bit_cast(v2i, r);
      if (kv < 32) {
        // after the transpose, value v of this lane is k = kr + v
        const int kr = KS * 16 + 8 * (lane >> 5) + 4 * h;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          unsigned x = static_cast<unsigned>(w[q]);
          if (kr + 2 * q >= kv) x &= 0xffff0000u;
          if (kr + 2 * q + 1 >= kv) x &= 0x0000ffffu;
          w[q] = static_cast<int>(x);
        }
      }
      half[h] = w;
    }
    return __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3);
  };

  auto read = [&](auto stage_tag, auto ks_tag, auto slot_tag, int kvalid) {
    constexpr int KS = decltype(ks_tag)::value, SL = decltype(slot_tag)::value;
    const uint8_t* sa = a_stage(stage_tag);
    const uint8_t* sb = b_stage(stage_tag);
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      if constexpr (AK) {
#pragma unroll
        for (int c = 0; c < LC; ++c) {
          af[SL][f][c] = *reinterpret_cast<const v4i*>(sa + a_wave_off + f * 32 * RSTEP + chunk_off[KS][c]);
          if (kvalid < KB) af[SL][f][c] = mask_bytes(af[SL][f][c], kvalid - chunk_of(KS, lane >> 5, c) * 16);
        }
      } else {
        af[SL][f][0] = read_mm(sa, PA, wm * TM + f * 32, ks_tag, kvalid / 2);
      }
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      if constexpr (BK) {
#pragma unroll
        for (int c = 0; c < LC; ++c) {
          bf[SL][f][c] = *reinterpret_cast<const v4i*>(sb + b_wave_off + f * 32 * RSTEP + chunk_off[KS][c]);
          if (kvalid < KB) bf[SL][f][c] = mask_bytes(bf[SL][f][c], kvalid - chunk_of(KS, lane >> 5, c) * 16);
        }
      } else {
        bf[SL][f][0] = read_mm(sb, PB, wn * TN + f * 32, ks_tag, kvalid / 2);
      }
    }
  };

  // MFMAs of sub-step KS on rows [I0, I1) of the wave tile from slot SL.
  auto mma = [&](auto ks_tag, auto slot_tag, auto i0_tag, auto i1_tag, const int (&scl)[NSC]) {
    constexpr int KS = decltype(ks_tag)::value, SL = decltype(slot_tag)::value;
    constexpr int I0 = decltype(i0_tag)::value, I1 = decltype(i1_tag)::value;
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        int s_a = 0, s_b = 0;
        if constexpr (T::SCALED) {
          s_a = scl[i];
          s_b = scl[FM + j];
        }
        acc[i][j] = T::template mma<KS>(af[SL][i], bf[SL][j], acc[i][j], s_a, s_b);
      }
  };

  // This lane's scale bytes for fragment row f (A rows first, then B),
  // zero-extended: fp4, blocks 2g and 2g+1 of the step for lane group g (one
  // per sub-step); MXFP8, block g.  In the tail step, blocks at or past K get
  // scale 1.0 (their data is zero).  gbuf is the step's group buffer, kq its
  // position in the group.
  auto scale_of = [&](const uint8_t* gbuf, int kq, int f, bool tail) -> int {
    const int row_all = f < FM ? wm * TM + f * 32 + (lane & 31) : BM + wn * TN + (f - FM) * 32 + (lane & 31);
    if constexpr (sps_of<T>() == 2) {
      int v = gbuf[row_all * SCW + 2 * kq + (lane >> 5)];
      if (tail && 2 * nkf + (lane >> 5) >= nkb) v = 127;
      return v;
    }
    int v = *reinterpret_cast<const uint16_t*>(gbuf + row_all * SCW + 4 * kq + 2 * (lane >> 5));
    if (tail) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (4 * nkf + 2 * (lane >> 5) + q >= nkb) v = (v & ~(0xff << (8 * q))) | (127 << (8 * q));
    }
    return v;
  };
  auto scales_of = [&](const uint8_t* gbuf, int kq, int (&scl)[NSC], bool tail) {
    if constexpr (T::SCALED) {
#pragma unroll
      for (int f = 0; f < NSC; ++f) scl[f] = scale_of(gbuf, kq, f, tail);
    } else {
      scl[0] = 0;
    }
  };

  using IFM = std::integral_constant<int, FM>;

  // One fragment of sub-step KS into fragment slot SL: R = 0 is A's first
  // row tile, 1 .. FN are B's column tiles, FN+1 .. are A's other row tiles
  // (the order the MFMAs of a phase consume them).
  auto read_one = [&](auto r_tag, auto ks_tag, auto slot_tag, auto stage_tag) {
    constexpr int R = decltype(r_tag)::value, KS = decltype(ks_tag)::value, SL = decltype(slot_tag)::value;
    constexpr bool IS_A = R == 0 || R > FN;
    constexpr int FI = R == 0 ? 0 : (IS_A ? R - FN : R - 1);
    if constexpr (IS_A) {
      if constexpr (AK) {
#pragma unroll
        for (int c = 0; c < LC; ++c)
          af[SL][FI][c] =
              *reinterpret_cast<const v4i*>(a_stage(stage_tag) + a_wave_off + FI * 32 * RSTEP + chunk_off[KS][c]);
      } else {
        af[SL][FI][0] = read_mm(a_stage(stage_tag), PA, wm * TM + FI * 32, ks_tag, 32);
      }
    } else {
      if constexpr (BK) {
#pragma unroll
        for (int c = 0; c < LC; ++c)
          bf[SL][FI][c] =
              *reinterpret_cast<const v4i*>(b_stage(stage_tag) + b_wave_off + FI * 32 * RSTEP + chunk_off[KS][c]);
      } else {
        bf[SL][FI][0] = read_mm(b_stage(stage_tag), PB, wn * TN + FI * 32, ks_tag, 32);
      }
    }
  };

  int scl[2][NSC];
  // One K-step; U is its position in the unrolled group, which fixes its
  // ring slot and fragment-slot parity at compile time.  Within a phase the
  // program order interleaves MFMAs, fragment reads and copies, and a hard
  // scheduling fence after each MFMA keeps that order: reads go out over
  // the first three quarters of the phase's MFMAs, copies over all of them.
  auto step = [&](auto uc, const int kt) {
    constexpr int U = decltype(uc)::value;
    constexpr int S = U % STAGES;  // ring slot of step kt
    constexpr int NEXT = (S + 1) % STAGES, ISSUE = (S + STAGES - 1) % STAGES;
    constexpr int PAR = U & 1;     // parity of kt (groups start at even kt)
    constexpr int SA = KSUB == 2 ? 0 : PAR;  // fragment slot used by phase A
    constexpr int SB = KSUB == 2 ? 1 : PAR;  // ... by phase B
    constexpr int SN = KSUB == 2 ? 0 : PAR ^ 1;  // ... filled for the next step
    using CUR = std::integral_constant<int, S>;
    const int* sc = scl[PAR];
    __builtin_amdgcn_sched_barrier(0);
    // ---- phase A: MFMAs of rows [0, RA) of the first sub-step; reads of the
    // second sub-step's fragments (two sub-steps per K-step)
    {
      // fp4: the next step's scales are read here, after this step's own
      // fragments (single stages: unless the next step starts a scale group,
      // whose buffer is only known to have landed after this step's barrier)
      constexpr bool SC_A = T::SCALED && (PAIR || (U + 1) % SG != 0);
      constexpr int NF_A = KSUB == 2 ? FM + FN : 0;
      constexpr int NM = RA * FN, NR = NF_A + (SC_A ? NSC : 0);
      constexpr int RM = NM * 3 / 4 > 0 ? NM * 3 / 4 : 1;
      const uint8_t* ng_a = nullptr;
      if constexpr (SC_A) ng_a = sgbuf(std::integral_constant<int, ((U + 1) / SG) % 2>{});
      // paired, even steps: the rest of the pair begun in the step before
      // (stages kt+2, kt+3)
      constexpr int PP = U + 2;
      constexpr int NV0 = (PAIR && U % 2 == 0) ? pair_first(PP) : 0;
      constexpr int NVA = (PAIR && U % 2 == 0) ? pair_count(PP) - NV0 : 0;
      const int s0 = kt + 2 < nkf ? kt + 2 : nkf - 1;
      __amdgpu_buffer_rsrc_t ra, rb;
      if constexpr (NVA > 0) pair_src(s0, ra, rb);
      static_for<NM>([&](auto tc) {
        constexpr int T_ = decltype(tc)::value, I = T_ / FN, J = T_ % FN;
        acc[I][J] = T::template mma<0>(af[SA][I], bf[SA][J], acc[I][J], T::SCALED ? sc[I] : 0,
                                       T::SCALED ? sc[FM + J] : 0);
        if constexpr (NR > 0 && T_ < RM) {
          static_for<((T_ + 1) * NR) / RM - (T_ * NR) / RM>([&](auto rc) {
            constexpr int R = (T_ * NR) / RM + decltype(rc)::value;
            if constexpr (R < NF_A) {
              read_one(std::integral_constant<int, R>{}, I1{}, I1{}, CUR{});
            } else if constexpr (SC_A) {
              scl[PAR ^ 1][R - NF_A] = scale_of(ng_a, (U + 1) % SG, R - NF_A, false);
            }
          });
        }
        static_for<((T_ + 1) * NVA) / NM - (T_ * NVA) / NM>([&](auto vc) {
          constexpr int V = NV0 + (T_ * NVA) / NM + decltype(vc)::value;
          issue_pair_one(std::integral_constant<int, V>{}, std::integral_constant<int, (PP % STAGES) / 2>{},
                         std::integral_constant<int, PP>{}, s0, ra, rb);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // ---- barrier: stage kt+1 visible, buffer kt-1 free
    wait_vm<younger(U)>();
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // ---- phase B: the remaining MFMAs; copies of stage kt+STAGES-1 into the
    // freed buffer; reads of the next step's first fragments and scales
    {
      // single: stage kt+STAGES-1; paired (odd steps): stages kt+3, kt+4
      const int nxt = kt + STAGES - 1 < nkf ? kt + STAGES - 1 : nkf - 1;
      __amdgpu_buffer_rsrc_t ra, rb;
      if constexpr (PAIR) {
        if constexpr (U % 2 != 0) pair_src(nxt, ra, rb);
      } else {
        step_src(nxt, ra, rb);
      }
      using NX = std::integral_constant<int, NEXT>;
      constexpr int NM = KSUB == 2 ? FM * FN : (FM - RA) * FN;
      constexpr int NF = FM + FN, NR = NF + ((T::SCALED && !PAIR && (U + 1) % SG == 0) ? NSC : 0);
      constexpr int RM = NM * 3 / 4 > 0 ? NM * 3 / 4 : 1;
      constexpr int P = U + STAGES - 1;  // position of the (first) stage issued here
      constexpr int NV = PAIR ? (U % 2 != 0 ? pair_first(U + 3) : 0) : issued_at(U);
      const uint8_t* ng = nullptr;  // the next step's scale group (fp4)
      if constexpr (T::SCALED) ng = sgbuf(std::integral_constant<int, ((U + 1) / SG) % 2>{});
      static_for<NM>([&](auto tc) {
        constexpr int T_ = decltype(tc)::value;
        constexpr int I = KSUB == 2 ? T_ / FN : RA + T_ / FN, J = T_ % FN;
        acc[I][J] = T::template mma<KSUB - 1>(af[SB][I], bf[SB][J], acc[I][J], T::SCALED ? sc[I] : 0,
                                              T::SCALED ? sc[FM + J] : 0);
        if constexpr (T_ < RM) {
          static_for<((T_ + 1) * NR) / RM - (T_ * NR) / RM>([&](auto rc) {
            // fp4 with single stages, when the next step starts a scale
            // group: its scales first, then the fragments in the order the
            // MFMAs consume them
            constexpr int R = (T_ * NR) / RM + decltype(rc)::value;
            constexpr int NS_ = NR - NF;
            if constexpr (R < NS_) {
              scl[PAR ^ 1][R] = scale_of(ng, (U + 1) % SG, R, false);
            } else {
              read_one(std::integral_constant<int, R - NS_>{}, I0{}, std::integral_constant<int, SN>{}, NX{});
            }
          });
        }
        static_for<((T_ + 1) * NV) / NM - (T_ * NV) / NM>([&](auto vc) {
          constexpr int V = (T_ * NV) / NM + decltype(vc)::value;
          if constexpr (PAIR) {
            issue_pair_one(std::integral_constant<int, V>{}, std::integral_constant<int, (ISSUE / 2)>{},
                           std::integral_constant<int, P>{}, nxt, ra, rb);
          } else {
            issue_one(std::integral_constant<int, V>{}, std::integral_constant<int, ISSUE>{},
                      std::integral_constant<int, P>{}, nxt, ra, rb);
          }
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  };


  // ---------------------------------------------------------- epilogue
  // The accumulators leave through LDS, one ER-row x 32-column block of the
  // wave tile at a time, so that every lane then owns 8 consecutive rows of
  // one column: C is read and D written in contiguous runs along M (whole
  // cache lines), and the per-element code is a loop, not one copy per
  // accumulator register.  When a staging area of its own fits next to the
  // ring, the next tile's first stages are already in flight meanwhile;
  // otherwise the blocks are staged in the (idle) ring.
  constexpr int LDS_WG = 163840 / OCC;  // 160 KiB of LDS per CU
  constexpr int RING = STAGES * STAGE + 2 * SC_BUF;  // with the scale group buffers
  constexpr int ER_OWN = (TM % 64 == 0 && RING + NW * 64 * 128 <= LDS_WG) ? 64
                         : (RING + NW * 32 * 128 <= LDS_WG)               ? 32
                                                                          : 0;
  constexpr bool EP_OWN = ER_OWN > 0;
  constexpr int RING_WPS_TM = STAGE / (TM * 128);  // waves per ring slot at the full wave-tile height
  constexpr int ER = EP_OWN ? ER_OWN : ((RING_WPS_TM > 0 && (NW + RING_WPS_TM - 1) / RING_WPS_TM <= STAGES) ? TM : 64);
  constexpr int EPB = ER * 32 * 4;  // staging bytes per wave
  constexpr int WPS = STAGE / EPB;  // waves per ring slot (ring staging)
  static_assert(EP_OWN || (WPS > 0 && (NW + WPS - 1) / WPS <= STAGES), "epilogue staging fits the ring");
  static_assert(TM % ER == 0 && ER % 32 == 0, "whole 32-row blocks");
  constexpr int LPC = ER / 8;                   // lanes per column (8 rows each)
  constexpr int CPI = 64 / LPC;                 // columns per iteration
  constexpr int XM = ER / 4 - 1 < 15 ? ER / 4 - 1 : 15;  // chunk swizzle mask (within the column)
  uint8_t* ep;
  if constexpr (EP_OWN) {
    ep = ep_area<NW * EPB>() + wave * EPB;
  } else {
    ep = slot(I0{});
    static_for<STAGES>([&](auto sc) {
      if (wave / WPS == decltype(sc)::value) ep = slot(sc);
    });
    ep += (wave % WPS) * EPB;
  }
  constexpr bool MXOUT = MXO && !T::INT;
  // MX output of one lane's 8-row run (rows m .. m+7 of column n; lo, hi
  // the staged accumulators): the epilogue values, the block's largest
  // magnitude over the 4 lanes that hold its 32 rows (consecutive lanes, the
  // first at a multiple of 4), then the element codes and, from the block's
  // first lane, its scale.  Called by every lane of the wave; lanes past M
  // or N take part in the maximum with nothing.
  auto mx_run = [&](const v4i lo, const v4i hi, const int64_t m, const int64_t n, void* const dst) {
    const bool valid = n < p.n && m < p.m;
    const int rows = valid ? static_cast<int>(p.m - m < 8 ? p.m - m : 8) : 0;
    const v4f lof = __builtin_bit_cast(v4f, lo), hif = __builtin_bit_cast(v4f, hi);
    float t[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) t[r] = p.alpha * (r < 4 ? lof[r] : hif[r - 4]);
    if (valid) {
      if (p.beta != 0.0f) {
        float cv[8];
        load8_f(p.c, p.c_type, n * p.ldc + m, rows, cv);
#pragma unroll
        for (int r = 0; r < 8; ++r) t[r] += p.beta * cv[r];
      }
      if (p.flags & EPI_BIAS) {
        float bv[8];
        load8_f(p.bias, p.bias_type, m, rows, bv);
#pragma unroll
        for (int r = 0; r < 8; ++r) t[r] += bv[r];
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      t[r] = activate(t[r], p.flags);
      if (r < rows) amax = __builtin_fmaxf(amax, __builtin_fabsf(t[r]));
    }
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
    if (!valid) return;
    const int emax = p.mx_out == MX_E2M1 ? 2 : (p.mx_out == MX_E4M3 ? 8 : 15);
    const int code = mx_scale_code(amax, emax);
    const float inv = __builtin_ldexpf(1.0f, 127 - code);  // 1 / 2^X, exact
    uint8_t* d8 = static_cast<uint8_t*>(dst);
    if (p.mx_out == MX_E2M1) {
      // two codes a byte along M, the even row in the low nibble
      uint32_t w = 0;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r < rows) w |= e2m1_code(t[r] * inv) << (4 * r);
      const int64_t off = (n * p.ldd + m) / 2;
      if (rows == 8 && (reinterpret_cast<uintptr_t>(d8 + off) & 3) == 0) {
        *reinterpret_cast<uint32_t*>(d8 + off) = w;
      } else {
        for (int q = 0; q < (rows + 1) / 2; ++q) d8[off + q] = static_cast<uint8_t>(w >> (8 * q));
      }
    } else {
      const float top = p.mx_out == MX_E4M3 ? 448.0f : 57344.0f;
      uint32_t w[2] = {0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = t[4 * h + r] * inv;
          v[r] = __builtin_fabsf(s) > top ? __builtin_copysignf(top, s) : s;
        }
        int lo2, hi2;
        if (p.mx_out == MX_E4M3) {
          lo2 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
          hi2 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo2, true);
        } else {
          lo2 = __builtin_amdgcn_cvt_pk_bf8_f32(v[0], v[1], 0, false);
          hi2 = __builtin_amdgcn_cvt_pk_bf8_f32(v[2], v[3], lo2, true);
        }
        w[h] = static_cast<uint32_t>(hi2);
      }
      const int64_t off = n * p.ldd + m;
      if (rows == 8 && (reinterpret_cast<uintptr_t>(d8 + off) & 7) == 0) {
        *reinterpret_cast<uint64_t*>(d8 + off) = (static_cast<uint64_t>(w[1]) << 32) | w[0];
      } else {
        for (int r = 0; r < rows; ++r) d8[off + r] = static_cast<uint8_t>(w[r / 4] >> (8 * (r % 4)));
      }
    }
    if ((m & 31) == 0) p.sfd[n * p.ld_sfd + (m >> 5)] = static_cast<uint8_t>(code);
  };

  auto epilogue_gen = [&](const int64_t em0, const int64_t en0, void* const dst) {
    int ln = lane;  // opaque copy, as in epilogue_vec below
    asm volatile("" : "+v"(ln));
    const int erow = (ln % LPC) * 8;
    static_for<(TM / ER) * FN>([&](auto pc) {
      // Block: rows ER*IR .. of the wave tile, column tile J, stored column by
      // column (ER*4 bytes each), 16-byte chunks XOR-swizzled by the column so
      // a write instruction spreads over the banks.
      constexpr int PS = decltype(pc)::value, IR = PS / FN, J = PS % FN;
      static_for<ER / 32>([&](auto iic) {
        constexpr int II = decltype(iic)::value;
        // whole-vector bit cast: a bit cast of one vector element reads element 0
        const v16i a = __builtin_bit_cast(v16i, acc[IR * (ER / 32) + II][J]);
        static_for<4>([&](auto gc) {
          constexpr int G = decltype(gc)::value;
          const int c = ln & 31, k = II * 8 + 2 * G + (ln >> 5);
          const v4i val = {a[4 * G], a[4 * G + 1], a[4 * G + 2], a[4 * G + 3]};
          *reinterpret_cast<v4i*>(ep + c * (ER * 4) + ((k ^ (c & XM)) << 4)) = val;
        });
      });
      // Lanes read what other lanes of the wave wrote: the LDS executes a
      // wave's accesses in order, so only the compiler must keep them in
      // program order (here and after the reads, before the next block).
      asm volatile("" ::: "memory");
      const int64_t m = em0 + wm * TM + IR * ER + erow;
      for (int it = 0; it < 32 / CPI; ++it) {
        const int c = it * CPI + ln / LPC;
        const int64_t n = en0 + wn * TN + J * 32 + c;
        const int ch = 2 * (ln % LPC);
        const v4i lo = *reinterpret_cast<const v4i*>(ep + c * (ER * 4) + ((ch ^ (c & XM)) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(ep + c * (ER * 4) + (((ch + 1) ^ (c & XM)) << 4));
        if (n < p.n && m < p.m) {
          const int rows = static_cast<int>(p.m - m < 8 ? p.m - m : 8);
          if constexpr (T::INT) {
            int t[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            if (p.beta != 0.0f) {
              int cv[8];
              load8_i(p.c, n * p.ldc + m, rows, cv);
  #pragma unroll
              for (int r = 0; r < 8; ++r) t[r] += cv[r];
            }
            if (p.flags & EPI_BIAS) {
              int bv[8];
              load8_i(p.bias, m, rows, bv);
  #pragma unroll
              for (int r = 0; r < 8; ++r) t[r] += bv[r];
            }
            if (p.flags & EPI_RELU) {
  #pragma unroll
              for (int r = 0; r < 8; ++r) t[r] = t[r] < 0 ? 0 : t[r];
            }
            store8_i(dst, n * p.ldd + m, t, rows);
          } else if (!MXOUT || p.mx_out == MX_NONE) {
            const v4f lof = __builtin_bit_cast(v4f, lo), hif = __builtin_bit_cast(v4f, hi);
            float t[8];
  #pragma unroll
            for (int r = 0; r < 8; ++r) t[r] = p.alpha * (r < 4 ? lof[r] : hif[r - 4]);
            if (p.beta != 0.0f) {
              float cv[8];
              load8_f(p.c, p.c_type, n * p.ldc + m, rows, cv);
  #pragma unroll
              for (int r = 0; r < 8; ++r) t[r] += p.beta * cv[r];
            }
            if (p.flags & EPI_BIAS) {
              float bv[8];
              load8_f(p.bias, p.bias_type, m, rows, bv);
  #pragma unroll
              for (int r = 0; r < 8; ++r) t[r] += bv[r];
            }
  #pragma unroll
            for (int r = 0; r < 8; ++r) t[r] = activate(t[r], p.flags);
            store8_f(dst, p.d_type, n * p.ldd + m, t, rows);
          }
        }
        if constexpr (MXOUT) {
          if (p.mx_out != MX_NONE) mx_run(lo, hi, m, n, dst);
        }
      }
      asm volatile("" ::: "memory");
    });
  };

  // Interior tiles whose D (and C, bias) rows allow 16-byte vectors along M
  // (host flag EPI_VEC, 16-bit C): the C and bias loads of a batch of EB
  // runs are all issued before the batch's first block is read, so a wave
  // waits for memory once per batch rather than once per block.  C and D are
  // addressed from the wave tile's corner: the lane's part in a VGPR, the
  // run's part in an SGPR.  The staging is pipelined: a block's runs are read
  // from LDS all at once, then the next block is written while this one is
  // computed and stored.
  //   LD: C or bias is read (else neither is);  BF: C, D and bias are bf16.
  // GELU takes the general path (its erf, copied into every run here, would
  // no longer be inlined).
  constexpr int NIT = 32 / CPI;         // iterations per block
  constexpr int NBLK = (TM / ER) * FN;  // blocks per wave tile
  constexpr int NU = NBLK * NIT;        // 8-row column runs per lane
  constexpr int EB = NU < 16 ? NU : 16; // runs per batch (4 VGPRs each)
  constexpr int BPB = EB / NIT;         // blocks per batch
  static_assert(NU % EB == 0 && EB % NIT == 0, "whole blocks per batch");
  auto stage_block = [&](auto ps_tag, int ln) {
    constexpr int PS = decltype(ps_tag)::value, IR = PS / FN, J = PS % FN;
    static_for<ER / 32>([&](auto iic) {
      constexpr int II = decltype(iic)::value;
      const v16i a = __builtin_bit_cast(v16i, acc[IR * (ER / 32) + II][J]);
      static_for<4>([&](auto gc) {
        constexpr int G = decltype(gc)::value;
        const int c = ln & 31, k = II * 8 + 2 * G + (ln >> 5);
        const v4i val = {a[4 * G], a[4 * G + 1], a[4 * G + 2], a[4 * G + 3]};
        *reinterpret_cast<v4i*>(ep + c * (ER * 4) + ((k ^ (c & XM)) << 4)) = val;
      });
    });
    // Lanes read what other lanes of the wave wrote: the LDS executes a
    // wave's accesses in order, so only the compiler must keep them in
    // program order.
    asm volatile("" ::: "memory");
  };
  auto epilogue_vec = [&](const int64_t em0, const int64_t en0, void* const dst, auto ld_tag, auto bf_tag) {
    constexpr bool LD = decltype(ld_tag)::value, BF = decltype(bf_tag)::value;
    // The lane index passes through an opaque copy so that the per-lane
    // addresses below are computed here rather than hoisted out of the tile
    // loop and kept live (spilled) through the main loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int erow = (ln % LPC) * 8;
    const int64_t tm0 = uniform64(em0 + wm * TM), tn0 = uniform64(en0 + wn * TN);
    const int cl = ln / LPC;  // the lane's column within an iteration
    const bool has_c = nonzero_f32(p.beta), has_bias = (p.flags & EPI_BIAS) != 0;
    const bool bias32 = p.bias_type == DT_F32, d32 = !BF && p.d_type == DT_F32;
    const unsigned c_bf = p.c_type == DT_BF16 ? ~0u : 0u, b_bf = p.bias_type == DT_BF16 ? ~0u : 0u;
    const unsigned d_bf = p.d_type == DT_BF16 ? ~0u : 0u, b32 = bias32 ? ~0u : 0u;
    // An absent C or bias (with the other present) is read through an empty
    // resource: its loads return zeros, so the loads do not depend on a
    // branch and neither does any wait for them.
    const auto rc = make_rsrc_u(static_cast<const uint16_t*>(p.c) + (has_c ? tn0 * p.ldc + tm0 : 0), has_c ? -1 : 0);
    const int ldcb = static_cast<int>(p.ldc) * 2;
    const uint32_t vc = static_cast<uint32_t>(cl * ldcb + erow * 2);
    const int bs = bias32 ? 4 : 2;
    const uint8_t* bbase = static_cast<const uint8_t*>(p.bias) + (has_bias ? tm0 * bs : 0);
    const auto rb = make_rsrc_u(bbase, has_bias ? -1 : 0), rb2 = make_rsrc_u(bbase, has_bias && bias32 ? -1 : 0);
    const int ds = d32 ? 4 : 2;
    const auto rd = make_rsrc_u(static_cast<uint8_t*>(dst) + (tn0 * p.ldd + tm0) * ds, -1);
    const int lddb = static_cast<int>(p.ldd) * ds;
    const uint32_t vd = static_cast<uint32_t>(cl * lddb + erow * ds);
    const float alpha = p.alpha, beta = p.beta;
    const int flags = p.flags;
    stage_block(std::integral_constant<int, 0>{}, ln);
    static_for<NU / EB>([&](auto bc) {
      constexpr int B0 = decltype(bc)::value * BPB;  // first block of the batch
      constexpr int IR0 = B0 / FN, NIR = (B0 + BPB - 1) / FN - IR0 + 1;
      v4i cv[EB];
      v4i bv[NIR][2];
      float bf[NIR][8];
      if constexpr (LD) {
        static_for<EB>([&](auto uc) {
          constexpr int U = decltype(uc)::value, PS = B0 + U / NIT, IT = U % NIT, IR = PS / FN, J = PS % FN;
          cv[U] = buf_load16(rc, vc, (J * 32 + IT * CPI) * ldcb + IR * ER * 2);
        });
        static_for<NIR>([&](auto irc) {
          constexpr int R = decltype(irc)::value;
          const uint32_t vo = static_cast<uint32_t>(erow * bs);
          bv[R][0] = buf_load16(rb, vo, (IR0 + R) * ER * bs);
          if constexpr (!BF) bv[R][1] = buf_load16(rb2, vo + 16, (IR0 + R) * ER * bs);
        });
      }
      static_for<BPB>([&](auto pc) {
        constexpr int PS = B0 + decltype(pc)::value, IR = PS / FN, J = PS % FN;
        if constexpr (LD) {
          if (PS == B0 || J == 0) {  // this row band's bias run, as floats (zeros if absent)
            float b16[8];
            unpack8(bv[IR - IR0][0], BF ? ~0u : b_bf, b16);
            if constexpr (BF) {
#pragma unroll
              for (int r = 0; r < 8; ++r) bf[IR - IR0][r] = b16[r];
            } else {
              const v4f b0 = __builtin_bit_cast(v4f, bv[IR - IR0][0]), b1 = __builtin_bit_cast(v4f, bv[IR - IR0][1]);
#pragma unroll
              for (int r = 0; r < 8; ++r)
                bf[IR - IR0][r] = __builtin_bit_cast(float, bsel(b32, __builtin_bit_cast(unsigned, r < 4 ? b0[r] : b1[r - 4]),
                                                                 __builtin_bit_cast(unsigned, b16[r])));
            }
          }
        }
        // this block's runs from LDS, then the next block into LDS
        v4f lo[NIT], hi[NIT];
        static_for<NIT>([&](auto ic) {
          constexpr int IT = decltype(ic)::value;
          const int c = IT * CPI + cl, ch = 2 * (ln % LPC);
          lo[IT] = __builtin_bit_cast(v4f, *reinterpret_cast<const v4i*>(ep + c * (ER * 4) + ((ch ^ (c & XM)) << 4)));
          hi[IT] = __builtin_bit_cast(v4f, *reinterpret_cast<const v4i*>(ep + c * (ER * 4) + (((ch + 1) ^ (c & XM)) << 4)));
        });
        asm volatile("" ::: "memory");
        if constexpr (PS + 1 < NBLK) stage_block(std::integral_constant<int, PS + 1>{}, ln);
        static_for<NIT>([&](auto ic) {
          constexpr int IT = decltype(ic)::value, U = (PS - B0) * NIT + IT;
          float t[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) t[r] = alpha * (r < 4 ? lo[IT][r] : hi[IT][r - 4]);
          if constexpr (LD) {
            float cf[8];
            unpack8(cv[U], BF ? ~0u : c_bf, cf);
#pragma unroll
            for (int r = 0; r < 8; ++r) t[r] = (t[r] + beta * cf[r]) + bf[IR - IR0][r];
          }
          if (flags & EPI_RELU) {  // gelu takes the general path
#pragma unroll
            for (int r = 0; r < 8; ++r) t[r] = t[r] > 0.0f ? t[r] : 0.0f;
          }
          const int so = (J * 32 + IT * CPI) * lddb + IR * ER * ds;
          if (d32) {
            buf_store16(__builtin_bit_cast(v4i, v4f{t[0], t[1], t[2], t[3]}), rd, vd, so);
            buf_store16(__builtin_bit_cast(v4i, v4f{t[4], t[5], t[6], t[7]}), rd, vd + 16, so);
          } else {
            buf_store16(pack8(t, BF ? ~0u : d_bf), rd, vd, so);
          }
        });
      });
    });
  };

  // The vector path needs registers for a batch of C runs next to the
  // staging: it is built where that fits without spilling (one workgroup per
  // CU, or the 128x128 two-workgroup variant with 16-byte copies).
  constexpr bool VEC_EPI = !T::INT && (OCC == 1 || (BM * BN <= 128 * 128 && LOADW == 16));
  auto epilogue = [&](const int64_t em0, const int64_t en0, void* const dst) {
    if constexpr (VEC_EPI) {
      if ((p.flags & EPI_VEC) && !(p.flags & EPI_GELU) && em0 + BM <= p.m && en0 + BN <= p.n) {
        const bool has_c = nonzero_f32(p.beta), has_bias = (p.flags & EPI_BIAS) != 0;
        const bool bf = (!has_c || p.c_type == DT_BF16) && p.d_type == DT_BF16 &&
                        (!has_bias || p.bias_type == DT_BF16);
        if (!bf) {
          epilogue_vec(em0, en0, dst, std::true_type{}, std::false_type{});
        } else if (has_c || has_bias) {
          epilogue_vec(em0, en0, dst, std::true_type{}, std::true_type{});
        } else {
          epilogue_vec(em0, en0, dst, std::false_type{}, std::true_type{});
        }
        return;
      }
    }
    epilogue_gen(em0, en0, dst);
  };

  // First stages of the current tile.
  auto prologue = [&]() {
    if constexpr (PAIR) {  // pairs (0, 1) and (2, 3): the whole ring
      if constexpr (T::SCALED) {  // scale group 0 (pair (2, 3) brings group 1)
#pragma unroll
        for (int t = 0; t < SC_LOADS; ++t) issue_scale(t, 0, sgbuf(I0{}));
      }
      issue_pair_full(0, I0{}, I0{});
      // pair (2, 3): its first part, as if issued in phase B of step -1
      __amdgpu_buffer_rsrc_t ra, rb;
      const int s2 = 2 < nkf ? 2 : nkf - 1;
      pair_src(s2, ra, rb);
      static_for<pair_first(2)>([&](auto vc) { issue_pair_one(vc, I1{}, std::integral_constant<int, 2>{}, s2, ra, rb); });
    } else {
      static_for<STAGES - 1>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        issue_full(S < nkf ? S : nkf - 1, std::integral_constant<int, S>{}, std::integral_constant<int, S>{});
      });
    }
  };

  // ---------------------------------------------------------- tile loop
  int id = static_cast<int>(blockIdx.y);
  setup(id);
  if (nkf > 0) prologue();
  for (bool first = true;; first = false) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};

    if (nkf > 0) {
      // Stage 0 landed.  After the first tile the previous epilogue's loads
      // and stores are in the count too, and vector-memory loads and stores
      // need not complete in order: wait for everything.
      if (first) {
        if constexpr (PAIR) {
          wait_vm<pair_first(2)>();  // the first part of pair (2, 3) may be in flight
        } else {
          wait_vm<younger(-1) + vm_of(STAGES - 2)>();  // stages 1 .. STAGES-2 may be in flight
        }
      } else {
        wait_vm<0>();
      }
      wg_barrier();
      if constexpr (T::SCALED) scales_of(sgbuf(I0{}), 0, scl[0], false);
      read(I0{}, I0{}, I0{}, KB);
      // Whole unrolled groups without per-step conditions (straight-line code
      // between loop edges), then the remaining steps.
      int kb = 0;
      for (; kb + UNROLL <= nkf; kb += UNROLL)
        static_for<UNROLL>([&](auto uc) { step(uc, kb + decltype(uc)::value); });
      static_for<UNROLL - 1>([&](auto uc) {
        if (kb + decltype(uc)::value < nkf) step(uc, kb + decltype(uc)::value);
      });
    }

    // The partial last K-step, if any: load it alone, then compute masked.
    if (nk > nkf) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // every buffer is free
      issue_partial(nkf);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      int sct[NSC];
      if constexpr (T::SCALED) {
        scales_of(((nkf / SG) & 1) ? sgbuf(I1{}) : sgbuf(I0{}), nkf % SG, sct, true);
      } else {
        sct[0] = 0;
      }
      const int kvalid = kbytes_u - nkf * KB;
      read(I0{}, I0{}, I0{}, kvalid);
      mma(I0{}, I0{}, I0{}, IFM{}, sct);
      if constexpr (KSUB == 2) {
        read(I0{}, I1{}, I1{}, kvalid);
        mma(I1{}, I1{}, I0{}, IFM{}, sct);
      }
    }

    __builtin_amdgcn_s_waitcnt(0);
    wg_barrier();  // every wave is done with the ring
    const int64_t em0 = m0, en0 = n0;
    void* const d_ep = d_unit;  // (setup of the next unit moves d_unit)
    const int next = id + static_cast<int>(gridDim.y);
    if constexpr (EP_OWN) {
      if (next < nunits) {
        setup(next);
        if (nkf > 0) prologue();
      }
      epilogue(em0, en0, d_ep);
    } else {
      epilogue(em0, en0, d_ep);
      if (next < nunits) {
        wg_barrier();  // the staging blocks in the ring are read
        setup(next);
        if (nkf > 0) prologue();
      }
    }
    if (next >= nunits) break;
    id = next;
  }
}

}  // namespace thl
