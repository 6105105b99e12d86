// gemm_kernels.hpp -- gfx950 GEMM kernels with a fused epilogue.
//
//   D = act(alpha * op(A) * op(B) + beta * C + bias[i])
//
// The tile hierarchy of the "CUTLASS" knowledge-base page ("The tile
// hierarchy"), built for CDNA4: a workgroup owns a BM x BN tile of D; its
// WM x WN wavefronts (64 lanes each) own (BM/WM) x (BN/WN) sub-tiles, each a
// grid of 32x32 MFMA tiles accumulated in registers.  K advances in steps of
// 128 bytes per operand row (64 fp16/bf16, 128 int8/fp8, 256 fp4 elements),
// so every operand format issues the same number of MFMA cycles per step.
//
// Global -> LDS (a3): direct-to-LDS loads (global_load_lds, 16 or 4 bytes a
// lane) into two swizzled stages; while stage s is consumed by the MFMAs,
// stage s+1 is in flight.  LDS -> registers (a4): each lane reads its 16-byte
// fragments from the swizzled rows.  Epilogue (a7): alpha/beta, bias,
// activation and conversion run on the accumulator registers, with C read
// and D written once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "index_maps.hpp"

namespace thl {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Operand families (one MFMA instruction each).
enum Family { FAM_F16 = 0, FAM_BF16 = 1, FAM_I8 = 2, FAM_FP8 = 3, FAM_FP4 = 4 };

// Element-type codes, equal to the public thl_dtype values.
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3, DT_I32 = 4 };
enum : int { EPI_BIAS = 1, EPI_RELU = 2, EPI_GELU = 4 };

struct GemmArgs {
  const uint8_t* a;  // K-major A: row i (of op(A)) at a + i*lda_bytes
  const uint8_t* b;  // K-major B: column j (of op(B)) at b + j*ldb_bytes
  const void* c;
  void* d;
  const void* bias;
  const uint8_t* sfa;  // fp4: E8M0 scales, row i block kb at sfa[i*ld_sfa + kb]
  const uint8_t* sfb;
  int64_t lda_bytes, ldb_bytes;
  int64_t ldc, ldd;  // elements
  int64_t ld_sfa, ld_sfb;
  int32_t m, n, k;  // k in elements
  int32_t kbytes;   // bytes of K per operand row
  int32_t tiles_m, tiles_n, group_m;
  float alpha, beta;  // alpha already holds the per-tensor fp8 scales
  int32_t flags;      // EPI_* bits
  int32_t c_type, d_type, bias_type;
};

// ------------------------------------------------------------ MFMA families
// Each family: LANE_CHUNKS 16-byte chunks per lane per MFMA, KSUB MFMAs per
// 128-byte K-step, the accumulator type, and the instruction.
template <int F>
struct Fam;

template <>
struct Fam<FAM_BF16> {
  static constexpr int LANE_CHUNKS = 1, KSUB = 4;
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
  static constexpr int LANE_CHUNKS = 1, KSUB = 4;
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
  static constexpr int LANE_CHUNKS = 1, KSUB = 4;
  static constexpr bool INT = true, SCALED = false;
  using Acc = v16i;
  template <int KS>
  static __device__ __forceinline__ Acc mma(const v4i* a, const v4i* b, Acc c, int, int) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], c, 0, 0, 0);
  }
};

template <>
struct Fam<FAM_FP8> {
  static constexpr int LANE_CHUNKS = 2, KSUB = 2;
  static constexpr bool INT = false, SCALED = false;
  using Acc = v16f;
  template <int KS>
  static __device__ __forceinline__ Acc mma(const v4i* a, const v4i* b, Acc c, int, int) {
    const v8i av = __builtin_shufflevector(a[0], a[1], 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i bv = __builtin_shufflevector(b[0], b[1], 0, 1, 2, 3, 4, 5, 6, 7);
    // Format 0 = E4M3 for both operands; no block scale (constant zero scale
    // operands select the unscaled instruction).
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
  }
};

template <>
struct Fam<FAM_FP4> {
  static constexpr int LANE_CHUNKS = 1, KSUB = 4;
  static constexpr bool INT = false, SCALED = true;
  using Acc = v16f;
  // Scale registers hold this lane's E8M0 bytes for the step: blocks 2*KS
  // and 2*KS+1 of the step alternate between lane halves, pre-shifted so the
  // lane's own byte sits at bit 0 (KS even) or bit 16 (KS odd) of the word.
  template <int KS>
  static __device__ __forceinline__ Acc mma(const v4i* a, const v4i* b, Acc c, int sa, int sb) {
    const v4i z = {0, 0, 0, 0};
    const v8i av = __builtin_shufflevector(a[0], z, 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i bv = __builtin_shufflevector(b[0], z, 0, 1, 2, 3, 4, 5, 6, 7);
    // Format 4 = E2M1 for both operands; opsel picks byte 0 or byte 2.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, (KS & 1) * 2, sa, (KS & 1) * 2, sb);
  }
};

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

// Store 4 consecutive rows m..m+3 of column n (rows >= `rows` skipped).
__device__ __forceinline__ void store4_f(void* d, int type, int64_t off, const float (&v)[4], int rows) {
  if (type == DT_F32) {
    float* p = static_cast<float*>(d) + off;
    if (rows >= 4 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      *reinterpret_cast<v4f*>(p) = v4f{v[0], v[1], v[2], v[3]};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < rows) p[i] = v[i];
    }
  } else if (type == DT_BF16) {
    __bf16* p = static_cast<__bf16*>(d) + off;
    __bf16 h[4] = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]), static_cast<__bf16>(v[2]),
                   static_cast<__bf16>(v[3])};
    if (rows >= 4 && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {
      *reinterpret_cast<v2i*>(p) = __builtin_bit_cast(v2i, h);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < rows) p[i] = h[i];
    }
  } else {  // DT_F16
    _Float16* p = static_cast<_Float16*>(d) + off;
    _Float16 h[4] = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]), static_cast<_Float16>(v[2]),
                     static_cast<_Float16>(v[3])};
    if (rows >= 4 && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {
      *reinterpret_cast<v2i*>(p) = __builtin_bit_cast(v2i, h);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < rows) p[i] = h[i];
    }
  }
}

// Direct global -> LDS load of W bytes per lane (W a literal the builtin accepts).
template <int W>
__device__ __forceinline__ void load_lds(const void* src, void* lds) {
  auto* l = (__attribute__((address_space(3))) void*)(lds);
  if constexpr (W == 16) {
    __builtin_amdgcn_global_load_lds(src, l, 16, 0, 0);
  } else {
    static_assert(W == 4, "16- or 4-byte lanes");
    __builtin_amdgcn_global_load_lds(src, l, 4, 0, 0);
  }
}

// ------------------------------------------------------------ the kernel

template <int F, int BM, int BN, int WM, int WN, int LOADW>
__global__ void __launch_bounds__(WM* WN * 64) gemm_kmajor_kernel(GemmArgs p) {
  using T = Fam<F>;
  using Acc = typename T::Acc;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, STAGE = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / (64 * LOADW), B_INSTR = B_BYTES / (64 * LOADW);
  constexpr int CHUNKS_PER_MFMA = 8 / T::KSUB;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole MFMA tiles");
  static_assert(A_INSTR % NW == 0 && B_INSTR % NW == 0, "copy instructions must split evenly over waves");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int wave = static_cast<int>(threadIdx.x) >> 6;
  const int wm = wave % WM, wn = wave / WM;
  int64_t tm, tn;
  maps::grouped_tile(maps::xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int nk = (p.kbytes + 127) >> 7;

  // One K-step of A and B, global -> LDS stage `buf`, as direct loads.
  auto issue = [&](int kt, int buf) {
    uint8_t* sa = smem + buf * STAGE;
    uint8_t* sb = sa + A_BYTES;
    const int64_t kbase = static_cast<int64_t>(kt) * 128;
#pragma unroll
    for (int j = 0; j < A_INSTR / NW; ++j) {
      const int base = (j * NW + wave) * 64 * LOADW;
      int64_t row, byte;
      maps::copy_source(base, lane, LOADW, &row, &byte);
      int64_t g = m0 + row;
      g = g < p.m ? g : p.m - 1;  // rows past M: any valid row (their outputs are not stored)
      int64_t kb = kbase + byte;
      kb = kb < p.kbytes ? kb : 0;  // bytes past K: any valid byte (masked before the MFMA)
      load_lds<LOADW>(p.a + g * p.lda_bytes + kb, sa + base);
    }
#pragma unroll
    for (int j = 0; j < B_INSTR / NW; ++j) {
      const int base = (j * NW + wave) * 64 * LOADW;
      int64_t row, byte;
      maps::copy_source(base, lane, LOADW, &row, &byte);
      int64_t g = n0 + row;
      g = g < p.n ? g : p.n - 1;
      int64_t kb = kbase + byte;
      kb = kb < p.kbytes ? kb : 0;
      load_lds<LOADW>(p.b + g * p.ldb_bytes + kb, sb + base);
    }
  };

  // fp4 block scales of this lane's rows for K-step kt: bytes 8*kt .. 8*kt+7
  // of each row, shifted so the lane half's byte is at bit 0 / bit 16.
  auto load_scales = [&](int kt, int (&sa)[FM][2], int (&sb)[FN][2]) {
    const int nkb = p.k >> 5;
    const int shift = 8 * (lane >> 5);
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      int64_t r = m0 + wm * TM + f * 32 + (lane & 31);
      r = r < p.m ? r : p.m - 1;
      const uint8_t* s = p.sfa + r * p.ld_sfa + 8 * kt;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        unsigned w = 0x7f7f7f7fu;
        if (8 * kt + 4 * h + 4 <= nkb && (reinterpret_cast<uintptr_t>(s + 4 * h) & 3) == 0) {
          w = *reinterpret_cast<const unsigned*>(s + 4 * h);
        } else {
          for (int q = 0; q < 4; ++q)
            if (8 * kt + 4 * h + q < nkb) w = (w & ~(0xffu << (8 * q))) | (static_cast<unsigned>(s[4 * h + q]) << (8 * q));
        }
        sa[f][h] = static_cast<int>(w >> shift);
      }
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      int64_t r = n0 + wn * TN + f * 32 + (lane & 31);
      r = r < p.n ? r : p.n - 1;
      const uint8_t* s = p.sfb + r * p.ld_sfb + 8 * kt;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        unsigned w = 0x7f7f7f7fu;
        if (8 * kt + 4 * h + 4 <= nkb && (reinterpret_cast<uintptr_t>(s + 4 * h) & 3) == 0) {
          w = *reinterpret_cast<const unsigned*>(s + 4 * h);
        } else {
          for (int q = 0; q < 4; ++q)
            if (8 * kt + 4 * h + q < nkb) w = (w & ~(0xffu << (8 * q))) | (static_cast<unsigned>(s[4 * h + q]) << (8 * q));
        }
        sb[f][h] = static_cast<int>(w >> shift);
      }
    }
  };

  Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};

  int sc_a[FM][2] = {}, sc_b[FN][2] = {};
  if (nk > 0) {
    issue(0, 0);
    if constexpr (T::SCALED) load_scales(0, sc_a, sc_b);
  }

  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of stage kt have landed
    __syncthreads();                // ... everyone's, and stage kt-1 is no longer read
    if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
    int cur_a[FM][2], cur_b[FN][2];
    if constexpr (T::SCALED) {
#pragma unroll
      for (int f = 0; f < FM; ++f) cur_a[f][0] = sc_a[f][0], cur_a[f][1] = sc_a[f][1];
#pragma unroll
      for (int f = 0; f < FN; ++f) cur_b[f][0] = sc_b[f][0], cur_b[f][1] = sc_b[f][1];
      if (kt + 1 < nk) load_scales(kt + 1, sc_a, sc_b);
    }
    const uint8_t* sa = smem + (kt & 1) * STAGE;
    const uint8_t* sb = sa + A_BYTES;
    const int kvalid = p.kbytes - kt * 128;

    auto step = [&](auto ks_tag) {
      constexpr int KS = decltype(ks_tag)::value;
      v4i af[FM][T::LANE_CHUNKS], bf[FN][T::LANE_CHUNKS];
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const int row = wm * TM + f * 32 + (lane & 31);
#pragma unroll
        for (int c = 0; c < T::LANE_CHUNKS; ++c) {
          const int chunk = KS * CHUNKS_PER_MFMA + (lane >> 5) * T::LANE_CHUNKS + c;
          af[f][c] = *reinterpret_cast<const v4i*>(sa + maps::lds_offset(row, chunk * 16));
          if (kvalid < 128) af[f][c] = mask_bytes(af[f][c], kvalid - chunk * 16);
        }
      }
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int row = wn * TN + f * 32 + (lane & 31);
#pragma unroll
        for (int c = 0; c < T::LANE_CHUNKS; ++c) {
          const int chunk = KS * CHUNKS_PER_MFMA + (lane >> 5) * T::LANE_CHUNKS + c;
          bf[f][c] = *reinterpret_cast<const v4i*>(sb + maps::lds_offset(row, chunk * 16));
          if (kvalid < 128) bf[f][c] = mask_bytes(bf[f][c], kvalid - chunk * 16);
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          int s_a = 0, s_b = 0;
          if constexpr (T::SCALED) {
            s_a = cur_a[i][KS >> 1];
            s_b = cur_b[j][KS >> 1];
          }
          acc[i][j] = T::template mma<KS>(af[i], bf[j], acc[i][j], s_a, s_b);
        }
    };
    step(std::integral_constant<int, 0>{});
    if constexpr (T::KSUB > 1) step(std::integral_constant<int, 1>{});
    if constexpr (T::KSUB > 2) {
      step(std::integral_constant<int, 2>{});
      step(std::integral_constant<int, 3>{});
    }
    (void)cur_a;
    (void)cur_b;
  }

  // ---------------------------------------------------------- epilogue
  // Straight-line code over every accumulator register (fully unrolled, no
  // early exits, so the accumulators stay in registers); rows and columns
  // past M and N are predicated off.
  static_for<FM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    static_for<FN>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int64_t n = n0 + wn * TN + j * 32 + (lane & 31);
      static_for<4>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        const int64_t m = m0 + wm * TM + i * 32 + 8 * g + 4 * (lane >> 5);
        if (n < p.n && m < p.m) {
          const int rows = static_cast<int>(p.m - m < 4 ? p.m - m : 4);
          if constexpr (T::INT) {
            int t[4];
            const int* cp = static_cast<const int*>(p.c) + n * p.ldc + m;
            const int* bp = static_cast<const int*>(p.bias) + m;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              int v = acc[i][j][4 * g + r];
              if (r < rows) {
                if (p.beta != 0.0f) v += cp[r];
                if (p.flags & EPI_BIAS) v += bp[r];
              }
              if ((p.flags & EPI_RELU) && v < 0) v = 0;
              t[r] = v;
            }
            int* dp = static_cast<int*>(p.d) + n * p.ldd + m;
            if (rows == 4 && (reinterpret_cast<uintptr_t>(dp) & 15) == 0) {
              *reinterpret_cast<v4i*>(dp) = v4i{t[0], t[1], t[2], t[3]};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (r < rows) dp[r] = t[r];
            }
          } else {
            float t[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float v = p.alpha * acc[i][j][4 * g + r];
              if (r < rows) {
                if (p.beta != 0.0f) v += p.beta * load_f(p.c, p.c_type, n * p.ldc + m + r);
                if (p.flags & EPI_BIAS) v += load_f(p.bias, p.bias_type, m + r);
              }
              t[r] = activate(v, p.flags);
            }
            store4_f(p.d, p.d_type, n * p.ldd + m, t, rows);
          }
        }
      });
    });
  });
}

}  // namespace thl
