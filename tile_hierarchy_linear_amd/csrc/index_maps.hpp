// index_maps.hpp -- the closed-form index functions the GEMM kernels use.
//
// Each is `__host__ __device__` so the library can evaluate it on the host
// (thl_kernel_index_map) and the tests can compare it, point by point, with
// the layout the Shape:Stride module computes for the same map -- the "host
// arithmetic against the layout algebra" check of the page "cute_layouts.cu"
// (gate 2), extended to every map the kernels rely on.
//
// Tile hierarchy ("CUTLASS" knowledge-base page, "The tile hierarchy"):
//   workgroup tile BM x BN  ->  wavefront tile (BM/WM) x (BN/WN)  ->  32x32 MFMA tiles.
// Operands are staged in LDS as rows of 64 bytes of K (one K-step), each row
// split into four 16-byte chunks whose order is XOR-swizzled per row.
#pragma once

#include <stdint.h>

#ifndef THL_HD
#define THL_HD __host__ __device__ __forceinline__
#endif

namespace thl {
namespace maps {

// ------------------------------------------------------------ a2: tiles
// Workgroups are handed to the 8 XCDs round-robin (workgroup w runs on XCD
// w % 8).  The remap makes each XCD own a contiguous range of logical tile
// ids, so tiles that share A/B panels share that XCD's L2:
//   logical = (w % 8) * (count / 8) + w / 8     when count % 8 == 0,
// and the identity otherwise.  As a layout: (8, count/8):(count/8, 1).
THL_HD int64_t xcd_remap(int64_t w, int64_t count) {
  if (count % 8 != 0) return w;
  return (w % 8) * (count / 8) + w / 8;
}

// Grouped raster: logical tile ids walk down a band of `group` tile rows
// (tile row fastest) before moving to the next tile column; bands follow one
// another.  With tm fastest this is the layout (group, tiles_n, tiles_m/group)
// : (1, tiles_m, group) onto the column-major tile index tm + tiles_m*tn, for
// tiles_m % group == 0; the last band is narrower otherwise.
THL_HD void grouped_tile(int64_t id, int64_t tiles_m, int64_t tiles_n, int64_t group, int64_t* tm,
                         int64_t* tn) {
  const int64_t band = group * tiles_n;
  const int64_t first = (id / band) * group;
  const int64_t rows = (tiles_m - first) < group ? (tiles_m - first) : group;
  const int64_t in_band = id % band;
  *tm = first + in_band % rows;
  *tn = in_band / rows;
}

// ------------------------------------------------------------ a3: LDS staging
// One K-step stages 64 bytes of K per operand row: four 16-byte chunks whose
// order is XOR-swizzled per row.  Chunk c of row r is stored in slot
// c ^ swz(r) with swz(r) = (r ^ (r >> 2)) & 3.  The MFMA fragment reads take
// one chunk from each of 32 consecutive rows (lane l: row l % 32; the two
// lane halves read different chunks).  Measured on gfx950 with 16 waves
// issuing such ds_read_b128, this swizzle streams about 230 B/clk per CU, the
// same as plain consecutive 16-byte reads; the earlier ((r >> 1) ^ (r >> 3))
// streamed 126 B/clk (two-way bank conflicts), although both put any 16
// consecutive rows on 16 distinct (row % 4, slot) pairs.  On the row-major
// (rows, 64) byte layout it is two XOR swizzles (b=2, m=4, s=2) and (b=2,
// m=4, s=4) composed on top.
constexpr int kStepBytes = 64;

THL_HD int swz(int64_t row) { return static_cast<int>((row ^ (row >> 2)) & 3); }

// Byte offset, inside one staged operand buffer, of byte `b` (0..63) of row `row`.
THL_HD int64_t lds_offset(int64_t row, int64_t b) {
  return row * kStepBytes + ((((b >> 4) ^ swz(row)) & 3) << 4) + (b & 15);
}

// Direct global->LDS loads write `loadw` bytes per lane at consecutive LDS
// addresses: lane `lane` of the instruction that starts at LDS byte `base`
// fills LDS bytes base + lane*loadw ... .  The lane therefore fetches the row
// and in-row byte that the inverse of lds_offset assigns to that LDS byte.
THL_HD void copy_source(int64_t base, int64_t lane, int64_t loadw, int64_t* row, int64_t* byte_in_row) {
  const int64_t off = base + lane * loadw;
  const int64_t r = off / kStepBytes;
  const int64_t slot = (off >> 4) & 3;
  *row = r;
  *byte_in_row = (((slot ^ swz(r)) & 3) << 4) | (off & 15);
}

// Paired stages.  With four stage buffers, stages 2j and 2j+1 share one
// buffer pair and are copied together, so that every copy instruction reads
// whole 128-byte lines (the vector L1 line; a 64-byte K-step alone fetches
// each line twice, once per step).  Rows are grouped by 8: group g is 1 KB,
// the group's 64 bytes of stage 2j followed by the same rows' 64 bytes of
// stage 2j+1.  Row r of a stage starts at byte r*64 + (r/8)*512 of the pair
// (+512 for the odd stage); the chunk swizzle inside a row is the one above.
THL_HD int64_t pair_row_offset(int64_t row) { return row * kStepBytes + (row >> 3) * 512; }

// Byte offset inside a buffer pair of byte `b` (0..63) of row `row` of the
// even (odd = 0) or odd (odd = 1) stage.
THL_HD int64_t pair_lds_offset(int64_t row, int64_t b, int64_t odd) {
  return pair_row_offset(row) + odd * 512 + (lds_offset(row, b) - row * kStepBytes);
}

// The 16-byte copy that fills 1 KB group `grp` (rows 8*grp .. 8*grp+7) of a
// pair: lane l fetches row 8*grp + (l%32)/4 and, within the 128 bytes of K
// the pair covers, byte 64*(l/32) plus the chunk that slot l%4 of that row
// holds.  Lanes l and l+32 take the two halves of one line.
THL_HD void pair_copy_source(int64_t grp, int64_t lane, int64_t* row, int64_t* byte_in_pair) {
  const int64_t r = 8 * grp + ((lane & 31) >> 2);
  *row = r;
  *byte_in_pair = 64 * (lane >> 5) + ((((lane & 3) ^ swz(r)) & 3) << 4);
}

// ------------------------------------------------------------ a4/a5: MFMA maps
// 32x32 MFMA operand fragment: lane l holds row l % 32 of the 32-row operand
// tile and `vals` consecutive K elements starting at (l / 32) * vals, where
// vals = 8 for 16-bit types (32x32x16), 16 for int8 (32x32x32) and 32 for fp4
// (32x32x64): the TV layout ((32,2),vals):((1, 32*vals), 32) onto the
// column-major (row + 32*k) tile index.
THL_HD void mfma32_operand(int64_t lane, int64_t v, int64_t vals, int64_t* row, int64_t* k) {
  *row = lane & 31;
  *k = (lane >> 5) * vals + v;
}

// 32x32 MFMA accumulator: register v of lane l is element
//   (row, col) = (8*(v/4) + 4*(l/32) + v%4, l % 32)
// i.e. the TV layout ((32,2),(4,4)):((32,4),(1,8)) onto the column-major
// (row + 32*col) tile index.  Each lane holds runs of 4 consecutive rows.
THL_HD void mfma32_acc(int64_t lane, int64_t v, int64_t* row, int64_t* col) {
  *row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
  *col = lane & 31;
}

// Small-M kernel, one 128-byte K unit of 16 operand rows (columns of B):
// byte j (0..31) of lane l is byte 16*(l/16) + j of the unit for j < 16 and
// 64 + 16*(l/16) + (j - 16) for j >= 16, of row l % 16: the TV layout
// ((16,4),(16,2)):((128,16),(1,64)) onto the row-major (k_byte + 128*row)
// index.  Each 16-byte half is one 16x16 MFMA's operand (16-bit, int8 and
// fp4 families: 16 bytes a lane); fp8 takes all 32 bytes in one 16x16x128.
// A lane's 16 bytes of fp4 are one 32-element scale block.
THL_HD void mfma16_operand(int64_t lane, int64_t j, int64_t* row, int64_t* kbyte) {
  *row = lane & 15;
  *kbyte = (j >> 4) * 64 + 16 * (lane >> 4) + (j & 15);
}

// 16x16 MFMA accumulator: register v of lane l is element
//   (row, col) = (4*(l/16) + v, l % 16)
// i.e. the TV layout ((16,4),4):((16,4),1) onto the column-major
// (row + 16*col) tile index: 4 consecutive rows of one column a lane.
THL_HD void mfma16_acc(int64_t lane, int64_t v, int64_t* row, int64_t* col) {
  *row = 4 * (lane >> 4) + v;
  *col = lane & 15;
}

// fp8 32x32x64 (f8f6f4 with 8-bit data): each lane supplies 32 bytes; the
// instruction reads them as K = 16*(l/32) + j for j < 16 and 32 + 16*(l/32) +
// (j - 16) for j >= 16.  The kernels load both operands with the same per-lane
// byte order, so any such fixed permutation of K cancels in the dot product.
THL_HD int64_t fp8_32x32_k_of(int64_t lane, int64_t j) {
  return j < 16 ? 16 * (lane >> 5) + j : 32 + 16 * (lane >> 5) + (j - 16);
}

// ------------------------------------------------------------ M-major operands
// An operand whose storage is contiguous along M (or N) -- opA = N, opB = T --
// is staged as k-rows: row k holds the tile's `pitch`/2 consecutive 16-bit
// elements of that k.  Its 32-byte blocks are XOR-swizzled by mm_swz(k), a
// permutation of 0..7 over k % 8: ((k & 3) << 1) | ((k >> 2) & 1).  Measured
// on gfx950 (16 waves of ds_read_b64_tr_b16 on 512-byte k-rows) it streams
// about 200 B/clk per CU against 123 B/clk for swizzling by k % 8 itself.
// pitch is a multiple of 256.
THL_HD int mm_swz(int64_t k) { return static_cast<int>(((k & 3) << 1) | ((k >> 2) & 1)); }

THL_HD int64_t mm_lds_offset(int64_t k, int64_t b, int64_t pitch) {
  return k * pitch + ((((b >> 5) ^ mm_swz(k))) << 5) + (b & 31);
}

// Inverse for the direct copies: the (k-row, byte within the row) that lane
// `lane` of the copy instruction starting at LDS byte `base` fetches.
THL_HD void mm_copy_source(int64_t base, int64_t lane, int64_t loadw, int64_t pitch, int64_t* k,
                           int64_t* byte_in_row) {
  const int64_t off = base + lane * loadw;
  const int64_t r = off / pitch;
  const int64_t pb = off % pitch;
  *k = r;
  *byte_in_row = ((((pb >> 5) ^ mm_swz(r))) << 5) | (pb & 31);
}

// The 8-byte chunk lane `lane` addresses for transposed read h (h = 0, 1) of a
// 32x32x16 16-bit MFMA operand: 4 consecutive rows m at one k, chosen so that
// after the transpose lane l holds row l % 32, k = 8*(l/32) + 4h + (0..3).
THL_HD void tr16_operand(int64_t lane, int64_t h, int64_t* k, int64_t* m) {
  *k = 8 * (lane >> 5) + 4 * h + ((lane & 15) >> 2);
  *m = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}

// Transposed 16-bit LDS read (ds_read_b64_tr_b16): inside each group of 16
// lanes, lane i receives element i % 4 of the 8-byte chunk that lane
// 4*v + i/4 of its group addressed, as its value v (v = 0..3).  Returned:
// (source lane within the group, element within that lane's chunk).
THL_HD void tr16_source(int64_t lane_in_group, int64_t v, int64_t* src_lane, int64_t* elem) {
  *src_lane = 4 * v + (lane_in_group >> 2);
  *elem = lane_in_group & 3;
}

}  // namespace maps
}  // namespace thl
