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

#include "gemm_args.hpp"
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

template <>
struct Fam<FAM_FP8> {
  static constexpr int LANE_CHUNKS = 2, KSUB = 1;
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
  static constexpr int LANE_CHUNKS = 1, KSUB = 2;
  static constexpr bool INT = false, SCALED = true;
  using Acc = v16f;
  // The scale register holds this lane's row's four E8M0 bytes for the step
  // (blocks 4kt .. 4kt+3), shifted right by 8*(lane/32) so that the lane's
  // block for sub-step KS (2KS + lane/32) sits in byte 2*KS.
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

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt low bits [3:0], high bits [15:14]; expcnt and
// lgkmcnt left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ------------------------------------------------------------ the kernel
//
// Pipeline (per wavefront, K-steps of 64 bytes per operand row, a ring of
// STAGES = 4 LDS buffers, copies always issued STAGES-1 steps ahead):
//
//   step kt, phase A:  first half of step kt's MFMAs; LDS reads of the
//                      fragments for the second half (from buffer kt).
//   barrier:           after this wave's copies of stage kt+1 have landed
//                      (only stage kt+2's may still be in flight); past it,
//                      stage kt+1 is visible and every wave has finished
//                      step kt-1, so buffer kt-1 is free.
//   step kt, phase B:  second half of step kt's MFMAs; LDS reads of step
//                      kt+1's first fragments; copies of stage kt+3 into
//                      the freed buffer.
//
// One barrier per step, placed so that the LDS latency of the next step's
// first fragments hides behind the current step's last MFMAs.  The copies
// past the last full step re-read the last full step (uniform, in bounds)
// so every step issues the same number of copies; a partial final K-step is
// loaded and computed after the loop with bytes past K masked to zero.
//
// Operand storage: AK (BK) true when op(A) rows (op(B) columns) are
// contiguous along K (opA = T, opB = N), staged as rows of 64 bytes of K;
// false when they are contiguous along M (N) -- 16-bit types only -- staged
// as 32 k-rows of the tile's M (N) extent and turned into K-contiguous
// fragments by two transposed 16-bit LDS reads each.
template <int F, int BM, int BN, int WM, int WN, int LOADW, int STAGES, int OCC, int SCW, bool AK, bool BK>
__global__ void __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
gemm_kernel(GemmArgs p) {
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
  // fp4 block scales travel with their stage: one dword (the 4 E8M0 bytes of
  // the K-step) per A and B row, copied with 4-byte lanes (scale rows must be
  // 4-byte aligned); the per-wave count is padded to a whole number with
  // copies into a dummy area so every wave issues the same.
  static_assert(SCW == 4, "scale copies are dwords");
  constexpr int SC_BYTES = T::SCALED ? (BM + BN) * 4 : 0;
  constexpr int SC_INSTR = T::SCALED ? (BM + BN) * 4 / (64 * SCW) : 0;
  constexpr int SC_LOADS = (SC_INSTR + NW - 1) / NW;
  constexpr int SC_PAD = T::SCALED ? 64 * SCW : 0;
  constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES + SC_PAD;
  constexpr int VM_STAGE = COPIES + SC_LOADS;  // vector-memory instructions per wave per stage
  static_assert(STAGE % 16 == 0, "stages stay 16-byte aligned");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole MFMA tiles");
  static_assert(A_LOADS * 64 * LOADW * NW == A_BYTES && B_LOADS * 64 * LOADW * NW == B_BYTES,
                "copies must split evenly over waves");
  static_assert(STAGES >= 3 && STAGES <= 5, "three to five stages");
  static_assert(VM_STAGE * (STAGES - 2) < 64, "vmcnt range");
  // Steps per unrolled loop body: ring slots and fragment-slot parities are
  // compile-time constants inside it.
  constexpr int UNROLL = (STAGES % 2 == 0) ? STAGES : 2 * STAGES;
  static_assert(KSUB == 2 || (KSUB == 1 && FM % 2 == 0), "a step splits into two halves");
  static_assert((AK && BK) || F == FAM_BF16 || F == FAM_F16, "M/N-major operands are 16-bit only");
  constexpr int PA = BM * 2, PB = BN * 2;  // k-row pitch of M- (N-) major stages
  static_assert(AK || PA % 256 == 0, "M-major k-rows are whole 256-byte bank windows");
  static_assert(BK || PB % 256 == 0, "N-major k-rows are whole 256-byte bank windows");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE];

  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int wm = wave % WM, wn = wave / WM;
  int64_t tm, tn;
  maps::grouped_tile(maps::xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int nk = (p.kbytes + KB - 1) / KB;  // K-steps, the last one possibly partial
  const int nkf = p.kbytes / KB;            // full K-steps

  // Per-tile operand bases (uniform), the per-step advance, and per-lane
  // 32-bit byte offsets of every copy this wave issues.  K-major: rows past M
  // (N) re-read the last valid row.  M-major: 16-byte chunks wholly past M
  // (N) re-read the tile's first chunk of that k-row.
  const uint8_t* a_tile = AK ? p.a + m0 * p.lda_bytes : p.a + m0 * 2;
  const uint8_t* b_tile = BK ? p.b + n0 * p.ldb_bytes : p.b + n0 * 2;
  const int64_t a_step = AK ? KB : 32 * p.lda_bytes;
  const int64_t b_step = BK ? KB : 32 * p.ldb_bytes;
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
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

  // fp4 scale copies: per lane, the source row base of each copy it issues.
  const int nkb = p.k >> 5;
  const uint8_t* sc_src[T::SCALED ? SC_LOADS : 1];
  int sc_dst[T::SCALED ? SC_LOADS : 1];
  if constexpr (T::SCALED) {
#pragma unroll
    for (int t = 0; t < SC_LOADS; ++t) {
      const int j = t * NW + wave;
      const int row_all = j < SC_INSTR ? j * 64 + lane : 0;
      if (row_all < BM) {
        const int64_t r = m0 + row_all < p.m ? m0 + row_all : p.m - 1;
        sc_src[t] = p.sfa + r * p.ld_sfa;
      } else {
        const int64_t r = n0 + (row_all - BM) < p.n ? n0 + (row_all - BM) : p.n - 1;
        sc_src[t] = p.sfb + r * p.ld_sfb;
      }
      sc_dst[t] = A_BYTES + B_BYTES + (j < SC_INSTR ? j * 64 * SCW : SC_BYTES);
    }
  }
  // Scale copies of step kt into a stage: bytes 4kt .. 4kt+3 of each row; an
  // offset at or past the row's last block reads the row's first dword (those
  // bytes are replaced before use).
  auto issue_scales = [&](int kt, uint8_t* stage) {
    if constexpr (T::SCALED) {
#pragma unroll
      for (int t = 0; t < SC_LOADS; ++t) {
        const int o = 4 * kt;
        load_lds<SCW>(sc_src[t] + (o < nkb ? o : 0), stage + sc_dst[t]);
      }
    }
  };

  // Copies of one full K-step into ring slot BUF: uniform base + 32-bit offset.
  auto issue_full = [&](int kt, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    uint8_t* sa = smem + BUF * STAGE;
    uint8_t* sb = sa + A_BYTES;
    issue_scales(kt, sa);
    const uint8_t* ak = a_tile + kt * a_step;
    const uint8_t* bk = b_tile + kt * b_step;
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) load_lds<LOADW>(ak + a_off[j], sa + (j * NW + wave) * 64 * LOADW);
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) load_lds<LOADW>(bk + b_off[j], sb + (j * NW + wave) * 64 * LOADW);
  };

  // The partial last K-step into slot 0: K-major bytes at or past K read the
  // row's first byte instead, M-major k-rows at or past K read the step's
  // first k-row (masked before the MFMAs).
  auto issue_partial = [&](int kt) {
    uint8_t* sa = smem;
    uint8_t* sb = sa + A_BYTES;
    const int64_t kofs = static_cast<int64_t>(kt) * KB;
    issue_scales(kt, sa);
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
      int64_t row, byte;
      const uint8_t* src;
      if constexpr (AK) {
        maps::copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, &row, &byte);
        src = a_tile + a_off[j] + (kofs + byte < p.kbytes ? kofs : -byte);
      } else {
        maps::mm_copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, PA, &row, &byte);
        const int64_t k = 32 * static_cast<int64_t>(kt) + row;
        src = a_tile + kt * a_step + a_off[j] - (k < p.k ? 0 : row * p.lda_bytes);
      }
      load_lds<LOADW>(src, sa + (j * NW + wave) * 64 * LOADW);
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
      int64_t row, byte;
      const uint8_t* src;
      if constexpr (BK) {
        maps::copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, &row, &byte);
        src = b_tile + b_off[j] + (kofs + byte < p.kbytes ? kofs : -byte);
      } else {
        maps::mm_copy_source((j * NW + wave) * 64 * LOADW, lane, LOADW, PB, &row, &byte);
        const int64_t k = 32 * static_cast<int64_t>(kt) + row;
        src = b_tile + kt * b_step + b_off[j] - (k < p.k ? 0 : row * p.ldb_bytes);
      }
      load_lds<LOADW>(src, sb + (j * NW + wave) * 64 * LOADW);
    }
  };

  Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};

  // Per-lane LDS offset of the chunk read for MFMA sub-step ks: fragment rows
  // differ by multiples of 32, which leave the swizzle unchanged, so one
  // offset per sub-step serves every fragment row (plus a constant).
  const int lrow = lane & 31;
  int chunk_off[KSUB][LC];
#pragma unroll
  for (int ks = 0; ks < KSUB; ++ks)
#pragma unroll
    for (int c = 0; c < LC; ++c)
      chunk_off[ks][c] = static_cast<int>(maps::lds_offset(lrow, (ks * CPM + (lane >> 5) * LC + c) * 16));
  const int a_wave_off = wm * TM * KB, b_wave_off = A_BYTES + wn * TN * KB;

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

  auto read = [&](const uint8_t* stage, auto ks_tag, auto slot_tag, int kvalid) {
    constexpr int KS = decltype(ks_tag)::value, SL = decltype(slot_tag)::value;
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      if constexpr (AK) {
#pragma unroll
        for (int c = 0; c < LC; ++c) {
          af[SL][f][c] = *reinterpret_cast<const v4i*>(stage + a_wave_off + f * 32 * KB + chunk_off[KS][c]);
          if (kvalid < KB) af[SL][f][c] = mask_bytes(af[SL][f][c], kvalid - (KS * CPM + (lane >> 5) * LC + c) * 16);
        }
      } else {
        af[SL][f][0] = read_mm(stage, PA, wm * TM + f * 32, ks_tag, kvalid / 2);
      }
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      if constexpr (BK) {
#pragma unroll
        for (int c = 0; c < LC; ++c) {
          bf[SL][f][c] = *reinterpret_cast<const v4i*>(stage + b_wave_off + f * 32 * KB + chunk_off[KS][c]);
          if (kvalid < KB) bf[SL][f][c] = mask_bytes(bf[SL][f][c], kvalid - (KS * CPM + (lane >> 5) * LC + c) * 16);
        }
      } else {
        bf[SL][f][0] = read_mm(stage + A_BYTES, PB, wn * TN + f * 32, ks_tag, kvalid / 2);
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

  // This lane's scale dword for each fragment row, read from a stage, shifted
  // right by 8*(lane/32) so sub-step KS finds its block in byte 2*KS.
  auto scales_of = [&](const uint8_t* stage, int (&scl)[NSC], bool tail) {
    if constexpr (T::SCALED) {
      const int shift = 8 * (lane >> 5);
#pragma unroll
      for (int f = 0; f < NSC; ++f) {
        const int row_all = f < FM ? wm * TM + f * 32 + (lane & 31) : BM + wn * TN + (f - FM) * 32 + (lane & 31);
        int v = *reinterpret_cast<const int*>(stage + A_BYTES + B_BYTES + row_all * 4);
        if (tail) {
          // blocks at or past K get scale 1.0 (their data is zero)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (4 * nkf + q >= nkb) v = (v & ~(0xff << (8 * q))) | (127 << (8 * q));
        }
        scl[f] = v >> shift;
      }
    } else {
      scl[0] = 0;
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using IFM = std::integral_constant<int, FM>;
  using IH = std::integral_constant<int, FM / 2>;

  if (nkf > 0) {
    // Prologue: stages 0 .. STAGES-2, then step 0's first fragments.
    static_for<STAGES - 1>([&](auto sc) {
      constexpr int S = decltype(sc)::value;
      issue_full(S < nkf ? S : nkf - 1, std::integral_constant<int, S>{});
    });
    wait_vm<(STAGES - 2) * VM_STAGE>();
    __syncthreads();
    read(smem, I0{}, I0{}, KB);

    for (int kb = 0; kb < nkf; kb += UNROLL) {
      static_for<UNROLL>([&](auto uc) {
        constexpr int U = decltype(uc)::value;
        constexpr int S = U % STAGES;  // ring slot of step kt
        constexpr int NEXT = (S + 1) % STAGES, ISSUE = (S + STAGES - 1) % STAGES;
        constexpr int PAR = U & 1;     // parity of kt (kb is even)
        const int kt = kb + U;
        if (kt < nkf) {
          const uint8_t* cur = smem + S * STAGE;
          int scl[NSC];
          scales_of(cur, scl, false);
          // ---- phase A
          if constexpr (KSUB == 2) {
            mma(I0{}, I0{}, I0{}, IFM{}, scl);
            read(cur, I1{}, I1{}, KB);
            static_for<FM * FN>([&](auto t) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              if constexpr (decltype(t)::value % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            });
          } else {
            mma(I0{}, std::integral_constant<int, PAR>{}, I0{}, IH{}, scl);
          }
          // ---- barrier: stage kt+1 visible, buffer kt-1 free
          wait_vm<(STAGES - 3) * VM_STAGE>();
          __syncthreads();
          // ---- phase B
          const int nxt = kt + STAGES - 1 < nkf ? kt + STAGES - 1 : nkf - 1;
          issue_full(nxt, std::integral_constant<int, ISSUE>{});
          if constexpr (KSUB == 2) {
            mma(I1{}, I1{}, I0{}, IFM{}, scl);
            read(smem + NEXT * STAGE, I0{}, I0{}, KB);
          } else {
            mma(I0{}, std::integral_constant<int, PAR>{}, IH{}, IFM{}, scl);
            read(smem + NEXT * STAGE, I0{}, std::integral_constant<int, PAR ^ 1>{}, KB);
          }
          constexpr int NM = (KSUB == 2) ? FM * FN : FM * FN / 2;
          constexpr int NR = (FM + FN) * LC;
          static_for<NM>([&](auto t) {
            constexpr int T_ = decltype(t)::value;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if constexpr ((T_ * NR) / NM != ((T_ + 1) * NR) / NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if constexpr ((T_ * VM_STAGE) / NM != ((T_ + 1) * VM_STAGE) / NM)
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          });
        }
      });
    }
  }

  // The partial last K-step, if any: load it alone, then compute masked.
  if (nk > nkf) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every buffer is free
    issue_partial(nkf);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int scl[NSC];
    scales_of(smem, scl, true);
    const int kvalid = p.kbytes - nkf * KB;
    read(smem, I0{}, I0{}, kvalid);
    mma(I0{}, I0{}, I0{}, IFM{}, scl);
    if constexpr (KSUB == 2) {
      read(smem, I1{}, I1{}, kvalid);
      mma(I1{}, I1{}, I0{}, IFM{}, scl);
    }
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
