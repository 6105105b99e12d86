// gemm_skinny.hpp -- the small-M GEMM kernel: M <= 64, K-major A and B.
//
// With one or a few rows of op(A), the product is a stream over B: every byte
// of B is used once, against a handful of A rows that every workgroup shares
// (they stay in L2).  The work is bound by HBM, not by the matrix cores, so
// this kernel stages nothing in LDS: it moves B from memory straight into
// MFMA operand registers, one whole 128-byte line per column per K unit, and
// spreads K over the wavefronts of a workgroup so that enough lines are in
// flight to cover HBM latency on every CU.  (The "CUTLASS" knowledge-base
// page's tile hierarchy still holds: workgroup tile (16 MT) x 16 of D,
// wavefront = one K slice of it, MFMA tile 16 x 16; the tiled kernels'
// smallest tile, 128 x 128, would run 127 rows of zeros through the matrix
// cores for M = 1 and give each workgroup 128 columns of B to stream.)
//
//   workgroup:  16 columns and MT sixteen-row tiles of D, KW wavefronts
//   wavefront:  K units [w*U/KW, (w+1)*U/KW) of U = ceil(K bytes / 128)
//   lane l:     row / column l % 16, bytes 16*(l/16) and 64 + 16*(l/16) of
//               each 128-byte unit (maps::mfma16_operand)
//   reduction:  the KW partial 16 x 16 tiles summed in LDS in wavefront order
//   epilogue:   alpha, C, bias, activation and rounding per element, as in
//               the tiled kernels
#pragma once

#include "gemm_kernels.hpp"

namespace thl {

// One 128-byte K unit: lane halves h = 0, 1 (16 bytes each) of A and B.
template <int F>
struct Skinny;

template <>
struct Skinny<FAM_BF16> {
  using Acc = v4f;
  static __device__ __forceinline__ Acc unit(const v4i (&a)[2], const v4i (&b)[2], Acc c, unsigned, unsigned) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[0]), __builtin_bit_cast(v8bf, b[0]), c, 0,
                                                0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[1]), __builtin_bit_cast(v8bf, b[1]), c,
                                                   0, 0, 0);
  }
};

template <>
struct Skinny<FAM_F16> {
  using Acc = v4f;
  static __device__ __forceinline__ Acc unit(const v4i (&a)[2], const v4i (&b)[2], Acc c, unsigned, unsigned) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a[0]), __builtin_bit_cast(v8h, b[0]), c, 0, 0,
                                               0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a[1]), __builtin_bit_cast(v8h, b[1]), c, 0,
                                                  0, 0);
  }
};

template <>
struct Skinny<FAM_I8> {
  using Acc = v4i;
  static __device__ __forceinline__ Acc unit(const v4i (&a)[2], const v4i (&b)[2], Acc c, unsigned, unsigned) {
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], b[0], c, 0, 0, 0);
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a[1], b[1], c, 0, 0, 0);
  }
};

// fp8: one 16x16x128 instruction takes a lane's 32 bytes; A and B arrive in
// the same per-lane byte order, so the order in which it reads K cancels.
// Format code 0 = E4M3, 1 = E5M2 (FA for A, FB for B).
template <int FA, int FB>
struct Skinny8 {
  using Acc = v4f;
  static __device__ __forceinline__ Acc unit(const v4i (&a)[2], const v4i (&b)[2], Acc c, unsigned, unsigned) {
    const v8i av = __builtin_shufflevector(a[0], a[1], 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i bv = __builtin_shufflevector(b[0], b[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, FA, FB, 0, 0, 0, 0);
  }
};
template <>
struct Skinny<FAM_FP8> : Skinny8<0, 0> {};
template <>
struct Skinny<FAM_E5M2> : Skinny8<1, 1> {};
template <>
struct Skinny<FAM_E4E5> : Skinny8<0, 1> {};
template <>
struct Skinny<FAM_E5E4> : Skinny8<1, 0> {};

template <>
struct Skinny<FAM_FP4> {
  using Acc = v4f;
  // Half h of the unit for lane group g is the 32-element block 4h + g of the
  // unit; sa / sb hold the lane's two E8M0 bytes (h = 0 in byte 0, h = 1 in
  // byte 1), and opsel picks the byte.
  static __device__ __forceinline__ Acc unit(const v4i (&a)[2], const v4i (&b)[2], Acc c, unsigned sa, unsigned sb) {
    const v4i z = {0, 0, 0, 0};
    const v8i a0 = __builtin_shufflevector(a[0], z, 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i b0 = __builtin_shufflevector(b[0], z, 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i a1 = __builtin_shufflevector(a[1], z, 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i b1 = __builtin_shufflevector(b[1], z, 0, 1, 2, 3, 4, 5, 6, 7);
    // Format 4 = E2M1 for both operands.
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, b0, c, 4, 4, 0, static_cast<int>(sa), 0,
                                                         static_cast<int>(sb));
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, b1, c, 4, 4, 1, static_cast<int>(sa), 1,
                                                            static_cast<int>(sb));
  }
};

// Lanes for rows past M and columns past N read at this offset, past the end
// of every operand resource: the buffer unit returns zeros for them without
// touching memory.  (Operand resources here span at most 64 rows or 16
// columns of at most 2^23 bytes, below 2^29, and per-unit offsets stay below
// 2^23, so no sum wraps.)
constexpr uint32_t kSkinnyOutside = 0x70000000u;
// Scalar offset of a K unit past a wavefront's range: also past the end of
// every operand resource (and below 2^32 with any lane offset).
constexpr int kSkinnyPast = 0x40000000;

template <class Acc>
__device__ __forceinline__ void store_tile(const GemmArgs& p, Acc sum, int64_t n0, int r_base);

// UN: K units per batch of loads (two batches in flight per wavefront).  On
// fp8 1 x 8192 x 8192, four wavefronts with two-unit batches stream B at
// about 6.8 TB/s once running; deeper batches were slower (up to 4 units of
// 8 in flight per wavefront measured).  MT: 16-row tiles of D per workgroup
// (M <= 16 * MT); every B operand register serves all MT of them, so B is
// still read once.
template <int F, int KW, int UN = 2, int MT = 1>
__global__ void __launch_bounds__(KW * 64) skinny_kernel(GemmArgs p) {
  offset_to_problem(p, blockIdx.y);
  using S = Skinny<F>;
  using Acc = typename S::Acc;
  constexpr bool SCALED = F == FAM_FP4;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  // The wavefront index read from lane 0, so that the K range and every
  // offset built from it stay scalar.
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int ncols = p.n - n0 < 16 ? static_cast<int>(p.n - n0) : 16;
  const int kb = p.kbytes;
  const int nunits = (kb + 127) >> 7;
  const int u_beg = wave * nunits / KW, u_end = (wave + 1) * nunits / KW;

  // Operand resources over A's m rows and B's ncols columns from n0, the
  // last row / column ending at the 16-byte boundary after its K-th byte
  // (the buffer unit range-checks whole dwords, so an exact end would zero
  // the dword that holds the last bytes; rows start 16-byte aligned, so the
  // rounded end stays in the last row's aligned 16 bytes, and the bytes
  // past K are masked before use).
  int64_t row, kbyte;
  maps::mfma16_operand(lane, 0, &row, &kbyte);
  const int kb16 = (kb + 15) & ~15;
  const auto ra = make_rsrc_n(p.a, static_cast<int>((p.m - 1) * p.lda_bytes + kb16));
  const auto rb = make_rsrc_n(p.b + n0 * p.ldb_bytes, static_cast<int>((ncols - 1) * p.ldb_bytes + kb16));
  uint32_t va[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    va[t] = row + 16 * t < p.m ? static_cast<uint32_t>((row + 16 * t) * p.lda_bytes + kbyte) : kSkinnyOutside;
  const uint32_t vb = row < ncols ? static_cast<uint32_t>(row * p.ldb_bytes + kbyte) : kSkinnyOutside;
  // fp4 scales: the row's (column's) 8 E8M0 bytes of the unit, blocks 8u ..
  // 8u+7 (rows start 16-byte aligned with lengths a multiple of 16, so an
  // 8-byte read at 8u < K/32 stays in the row).
  const int nkb = p.k >> 5;
  __amdgpu_buffer_rsrc_t rsa = ra, rsb = rb;
  uint32_t vsa[MT] = {}, vsb = 0;
  if constexpr (SCALED) {
    rsa = make_rsrc_n(p.sfa, static_cast<int>((p.m - 1) * p.ld_sfa + ((nkb + 15) & ~15)));
    rsb = make_rsrc_n(p.sfb + n0 * p.ld_sfb, static_cast<int>((ncols - 1) * p.ld_sfb + ((nkb + 15) & ~15)));
#pragma unroll
    for (int t = 0; t < MT; ++t)
      vsa[t] = row + 16 * t < p.m ? static_cast<uint32_t>((row + 16 * t) * p.ld_sfa) : kSkinnyOutside;
    vsb = row < ncols ? static_cast<uint32_t>(row * p.ld_sfb) : kSkinnyOutside;
  }
  const int g = lane >> 4;
  Acc acc[MT] = {};

  struct Unit {
    v4i a[MT][2], b[2];
    v2i sa[MT], sb;  // fp4: the 8 E8M0 bytes of the unit's blocks
  };
  // Unit u's loads; a unit at or past the wave's end reads zeros (offset past
  // every resource) and adds nothing.  No loaded value is touched here, so
  // nothing waits for memory before the MFMAs that need it.
  auto load = [&](int u, Unit& x) {
    const int so = u < u_end ? (u << 7) : kSkinnyPast;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      x.b[h] = buf_load16(rb, vb + 64 * h, so);
#pragma unroll
      for (int t = 0; t < MT; ++t) x.a[t][h] = buf_load16(ra, va[t] + 64 * h, so);
    }
    if constexpr (SCALED) {
      const int ss = u < u_end ? (u << 3) : kSkinnyPast;
#pragma unroll
      for (int t = 0; t < MT; ++t)
        x.sa[t] = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(rsa, vsa[t], ss, 0));
      x.sb = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(rsb, vsb, ss, 0));
    }
  };
  // Unit u's MFMAs.  In a unit that runs past K the bytes past K are zeroed
  // and scale blocks past K/32 read as 2^0 (their data is zero; a NaN code
  // in row padding would otherwise poison the sum).
  // byte 0: block 8u + g (half 0), byte 1: block 8u + 4 + g (half 1)
  auto scale_pair = [&](v2i w) -> unsigned {
    const unsigned sh = 8u * static_cast<unsigned>(g);
    return ((static_cast<unsigned>(w[0]) >> sh) & 0xffu) | (((static_cast<unsigned>(w[1]) >> sh) & 0xffu) << 8);
  };
  auto use = [&](int u, Unit& x) {
    const int so = u << 7;
    unsigned sa[MT] = {}, sb = 0;
    if constexpr (SCALED) {
#pragma unroll
      for (int t = 0; t < MT; ++t) sa[t] = u < u_end ? scale_pair(x.sa[t]) : 0x7f7fu;
      sb = u < u_end ? scale_pair(x.sb) : 0x7f7fu;  // zero data past the range: unit scales
    }
    if (u < u_end && so + 128 > kb) {  // the last, partial unit (uniform branch)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int valid = kb - (so + 64 * h + 16 * g);
        x.b[h] = mask_bytes(x.b[h], valid);
#pragma unroll
        for (int t = 0; t < MT; ++t) x.a[t][h] = mask_bytes(x.a[t][h], valid);
      }
      if constexpr (SCALED) {
        const int blk = 8 * u + g;
        const unsigned keep = (blk >= nkb ? 0u : 0xffu) | (blk + 4 >= nkb ? 0u : 0xff00u);
        const unsigned unit1 = (blk >= nkb ? 127u : 0u) | (blk + 4 >= nkb ? 127u << 8 : 0u);
#pragma unroll
        for (int t = 0; t < MT; ++t) sa[t] = (sa[t] & keep) | unit1;
        sb = (sb & keep) | unit1;
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = S::unit(x.a[t], x.b, acc[t], sa[t], sb);
  };

  // Two batches of UN units in flight: batch j+1's loads go out before batch
  // j's MFMAs.
  Unit x0[UN], x1[UN];
  const int nbatch = (u_end - u_beg + UN - 1) / UN;
#pragma unroll
  for (int i = 0; i < UN; ++i) load(u_beg + i, x0[i]);
  for (int j = 0; j < nbatch; j += 2) {
    const int u = u_beg + j * UN;
#pragma unroll
    for (int i = 0; i < UN; ++i) load(u + UN + i, x1[i]);
#pragma unroll
    for (int i = 0; i < UN; ++i) use(u + i, x0[i]);
#pragma unroll
    for (int i = 0; i < UN; ++i) load(u + 2 * UN + i, x0[i]);
#pragma unroll
    for (int i = 0; i < UN; ++i) use(u + UN + i, x1[i]);
  }

  // Sum the KW partial tiles in wavefront order (the same order for every
  // element, so the result does not depend on timing).
  __shared__ __attribute__((aligned(16))) v4i part[KW][MT][64];
#pragma unroll
  for (int t = 0; t < MT; ++t) part[wave][t][lane] = __builtin_bit_cast(v4i, acc[t]);
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    Acc sum = __builtin_bit_cast(Acc, part[0][t][lane]);
#pragma unroll
    for (int w = 1; w < KW; ++w) sum += __builtin_bit_cast(Acc, part[w][t][lane]);
    store_tile(p, sum, n0, 16 * t);
  }
}

// Epilogue of one 16 x 16 tile whose first row is r_base: lane l holds rows
// r_base + 4*(l/16) .. +3 of column n0 + l % 16.
template <class Acc>
__device__ __forceinline__ void store_tile(const GemmArgs& p, Acc sum, int64_t n0, int r_base) {
  constexpr bool INT = std::is_same<Acc, v4i>::value;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  int64_t r0, c0;
  maps::mfma16_acc(lane, 0, &r0, &c0);
  r0 += r_base;
  const int64_t n = n0 + c0;
  if (n >= p.n || r0 >= p.m) return;
  const int rows = p.m - r0 < 4 ? static_cast<int>(p.m - r0) : 4;
  if constexpr (INT) {
    int t[8] = {sum[0], sum[1], sum[2], sum[3], 0, 0, 0, 0};
    if (p.beta != 0.0f) {
      int cv[8];
      load8_i(p.c, n * p.ldc + r0, rows, cv);
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] += cv[r];
    }
    if (p.flags & EPI_BIAS) {
      int bv[8];
      load8_i(p.bias, r0, rows, bv);
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] += bv[r];
    }
    if (p.flags & EPI_RELU) {
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = t[r] < 0 ? 0 : t[r];
    }
    store8_i(p.d, n * p.ldd + r0, t, rows);
  } else {
    float t[8] = {p.alpha * sum[0], p.alpha * sum[1], p.alpha * sum[2], p.alpha * sum[3], 0.0f, 0.0f, 0.0f, 0.0f};
    if (p.beta != 0.0f) {
      float cv[8];
      load8_f(p.c, p.c_type, n * p.ldc + r0, rows, cv);
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] += p.beta * cv[r];
    }
    if (p.flags & EPI_BIAS) {
      float bv[8];
      load8_f(p.bias, p.bias_type, r0, rows, bv);
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] += bv[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] = activate(t[r], p.flags);
    store8_f(p.d, p.d_type, n * p.ldd + r0, t, rows);
  }
}

}  // namespace thl
