// Device-friendly layouts of the 4-bit operands and their scales.
//
// K is cut into steps of 128 elements (64 bytes of codes per row).  Codes
// are stored in 1 KB units of 16 rows x one step, units ordered [row / 16]
// [step], so every direct-to-LDS load moves one contiguous kilobyte.  Inside
// a unit, 16-byte slot p = 4 (row % 16) + q holds chunk q ^ chunk_swz(row)
// of that row's 64 bytes: the XOR swizzle the GEMM kernels read LDS with.
//
// Scale records (16 bytes per row and 4 steps) are stored in 1 KB units of
// 64 rows, ordered [row / 64][4-step group].  INT4 weight scales are stored
// in 2 KB units of 128 rows x 4 steps, ordered [row / 128][4-step group];
// inside a unit [4-row block][step % 4][row % 4][group of 64] fp16.
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

// fp16 index of the INT4 weight scale of row n, step t, 64-group G (0, 1) of the step
SVDQ_HD inline size_t int4_wscale_index(int n, int t, int G, int ks4) {
  return ((size_t)(n >> 7) * ks4 + (t >> 2)) * 1024 + (size_t)((n & 127) >> 2) * 32 + (t & 3) * 8 + (n & 3) * 2 + G;
}
SVDQ_HD inline size_t int4_wscale_bytes(int rows, int ks4) { return (size_t)((rows + 127) / 128) * ks4 * 2048; }

}  // namespace svdq

#endif
