// Device-friendly layouts of the 4-bit operands and their scales.
//
// K is cut into steps of 128 elements (64 bytes of codes per row).  Codes
// are stored in 1 KB units of 16 rows x one step, units ordered [row / 16]
// [step], so every direct-to-LDS load moves one contiguous kilobyte.  Inside
// a unit, 16-byte slot p = 4 (row % 16) + q holds chunk q ^ chunk_swz(row)
// of that row's 64 bytes: the XOR swizzle the GEMM kernels read LDS with.
//
// Scale records (16 bytes per row and 4 steps; MXFP4) are stored in 1 KB
// units of 64 rows, ordered [row / 64][4-step group].  INT4 codes and scales
// have layouts of their own (below).
#ifndef SVDQ_LAYOUT_H
#define SVDQ_LAYOUT_H

#include <cstddef>
#include <cstdint>

#if defined(__HIPCC__)
#define SVDQ_HD __host__ __device__
#else
#define SVDQ_HD
#endif

namespace svdq {

// chunk_swz(row) = row bit 1 + 2 x row bit 3.  A 16-byte LDS read of a wave
// is served 16 lanes per cycle, lanes grouped by (lane bit 5, parity of lane
// bits 2-4), and two lanes of a group conflict when their addresses agree in
// bits 4-7; with this swizzle the GEMM kernels' fragment reads (16 rows at
// one chunk, lanes 16 g + i reading row i, chunk g; consecutive rows or rows
// 8 j + i, i < 4) give every group 16 distinct slots.
SVDQ_HD inline int chunk_swz(int row) { return ((row >> 1) & 1) | ((row >> 2) & 2); }

// byte b (0..63) of step t of row `row`
SVDQ_HD inline size_t code_offset(int row, int t, int b, int steps) {
  return ((size_t)(row >> 4) * steps + t) * 1024 +
         (size_t)(4 * (row & 15) + ((b >> 4) ^ chunk_swz(row & 31))) * 16 + (b & 15);
}
SVDQ_HD inline size_t code_bytes(int rows, int steps) { return (size_t)((rows + 15) / 16) * steps * 1024; }

// byte j (0..15) of the scale record of row `row` for 4-step group q.  A
// row's record is 4 dwords; dword d of row r sits at dword 64 (r % 64 / 16)
// + 16 d + r % 16 of the 1 KB unit, so the GEMM's scale read (64 lanes:
// 16 rows x dword g) covers 256 contiguous bytes.
SVDQ_HD inline size_t scale_record_offset(int row, int q, int j, int ks4) {
  return ((size_t)(row >> 6) * ks4 + q) * 1024 +
         (size_t)(64 * ((row & 63) >> 4) + 16 * (j >> 2) + (row & 15)) * 4 + (j & 3);
}
// MXFP4 weight scale records hold their rows in the order the GEMM's weight
// fragments read them: inside each 64-row block, row 32 p + 8 j + 4 h + i
// (i < 4, j < 4, h < 2) is stored as row 16 (2 p + h) + 4 j + i.
SVDQ_HD inline int wrec_row(int row) {
  const int r = row & 63;
  return (row & ~63) | (16 * (2 * (r >> 5) + ((r >> 2) & 1)) + 4 * ((r >> 3) & 3) + (r & 3));
}
SVDQ_HD inline size_t scale_record_bytes(int rows, int ks4) { return (size_t)((rows + 63) / 64) * ks4 * 1024; }

// ---- INT4 on the device.  Codes -7..7 are stored as FP6 E2M3 values (exact
// for these integers), the operand type of the scaled 32x32x64 MFMA, whose
// K extent is one 64-element group.  A 128-element step of a row holds four
// 32-element slices s = 2 G + h (elements 64 G + 32 h .. +32); a slice is 32
// six-bit codes packed in 6 dwords, element j at bits 6 j.  Dwords 0-3 of
// slice s ("main") sit in the codes layout above, 16-byte slot
// 4 (row % 16) + (s ^ i4_swz(row)); dwords 4-5 ("tail") in 1 KB units of 32
// rows x one step ordered [row / 32][step], at unit byte 256 s + 8 (row % 32).
//
// i4_swz(row) = row bits 2-3: the 32x32 MFMA's fragment read (lane l: row
// l % 32, or its out-feature permutation, at slot 2 G + l / 32) then gives
// every 16-lane LDS group 16 distinct 16-byte slots.
SVDQ_HD inline int i4_swz(int row) { return (row >> 2) & 3; }
SVDQ_HD inline size_t i4_main_offset(int row, int t, int s, int steps) {
  return ((size_t)(row >> 4) * steps + t) * 1024 + (size_t)(4 * (row & 15) + (s ^ i4_swz(row))) * 16;
}
SVDQ_HD inline size_t i4_tail_offset(int row, int t, int s, int steps) {
  return ((size_t)(row >> 5) * steps + t) * 1024 + (size_t)256 * s + 8 * (row & 31);
}
SVDQ_HD inline size_t i4_tail_bytes(int rows, int steps) { return (size_t)((rows + 31) / 32) * steps * 1024; }
// INT4 scales: 512-byte units of 128 rows x one step ordered [row / 128][step].
// Activations: dword row % 128 is the fp16 pair of the step's groups 2t
// (low half) and 2t + 1; weights: fp16 index 128 G + row % 128.
SVDQ_HD inline size_t i4_scale_bytes(int rows, int steps) { return (size_t)((rows + 127) / 128) * steps * 512; }
SVDQ_HD inline size_t i4_xscale_offset(int row, int t, int G, int steps) {
  return ((size_t)(row >> 7) * steps + t) * 512 + 4 * (row & 127) + 2 * G;
}
SVDQ_HD inline size_t i4_wscale_offset(int row, int t, int G, int steps) {
  return ((size_t)(row >> 7) * steps + t) * 512 + 2 * (128 * G + (row & 127));
}
// FP6 E2M3 code of an INT4 value (sign bit 5, exponent bits 3-4 with bias
// 1, mantissa bits 0-2): 1 = 1.0 x 2^0, 3 = 1.5 x 2^1, 5 = 1.25 x 2^2, ...
SVDQ_HD inline uint8_t e2m3_of_int4(int q) {
  const int a = q < 0 ? -q : q;
  const uint8_t mag = a == 0 ? 0 : a == 1 ? 0x08 : a == 2 ? 0x10 : a == 3 ? 0x14 : a == 4 ? 0x18 : a == 5 ? 0x1A
                    : a == 6 ? 0x1C : 0x1E;
  return (uint8_t)((q < 0 ? 0x20 : 0) | mag);
}

}  // namespace svdq

#endif
