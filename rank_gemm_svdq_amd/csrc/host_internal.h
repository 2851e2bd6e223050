// Internal declarations shared by the host-side translation units of the
// library (not part of the ABI).
#pragma once

#include <cstddef>
#include <cstdint>
#include <functional>
#include <vector>

#include "../../include/svdq.h"
#include "layout.h"

namespace svdq {

constexpr int kStep = 128;  // K elements per main-loop step of both kernels

inline int group_size(int fmt) { return fmt == SVDQ_INT4_G64 ? 64 : 32; }   // the 4-bit formats
inline bool is_w8(int fmt) { return fmt == SVDQ_W8A8; }
// code steps of 64 bytes per row: 128 elements (4-bit) or 64 (8-bit)
inline int32_t code_steps(int32_t K, int fmt) { return is_w8(fmt) ? K / 64 : K / 128; }
// canonical buffers: codes [rows, K/2] (4-bit) or [rows, K] (8-bit); scales
// [rows, K/64] fp16, [rows, K/32] E8M0 or [rows] fp32
inline size_t canon_code_bytes(int64_t rows, int32_t K, int fmt) {
  return is_w8(fmt) ? (size_t)rows * K : (size_t)rows * (K / 2);
}
inline size_t canon_scale_bytes(int64_t rows, int32_t K, int fmt) {
  return fmt == SVDQ_INT4_G64 ? (size_t)rows * (K / 64) * 2 : fmt == SVDQ_MXFP4_G32 ? (size_t)rows * (K / 32)
                                                                                   : (size_t)rows * 4;
}
inline int32_t rank_pad(int32_t rank) { return (rank + 31) / 32 * 32; }
inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Kernel-layout geometry (documented in the device source and DESIGN notes)
struct Geometry {
  int32_t K, N, rank, rpad, fmt, steps, ks4, csteps;   // csteps: 64-byte code steps per row
  size_t wq_bytes, ws_bytes, l1k_bytes, l2k_bytes;
};
bool geometry(int32_t K, int32_t N, int32_t rank, int32_t fmt, Geometry* g);
bool valid_kn(int32_t K, int32_t N);
bool valid_rank(int32_t rank);
bool valid_fmt(int32_t fmt);
int32_t choose_zsplit(int32_t M, int32_t K);

// Byte position of canonical element k (0..127) inside a 64-byte INT4 step.
inline int int4_step_byte(int k) {
  const int G = k >> 6, r = k & 63, g = r >> 4, j = r & 15;
  return 16 * g + 8 * G + (j >> 1);
}

// Scalar conversions (round to nearest even).
uint16_t bf16_from_double(double x);
double double_from_bf16(uint16_t h);
uint16_t half_from_float(float x);
float float_from_half(uint16_t h);

// Quantizers of one group, shared by the weight packer and the unpack helper.
void quant_int4_group(const float* x, uint8_t* nib /*64 nibble values*/, uint16_t* scale_bits);
void quant_mxfp4_group(const float* x, uint8_t* nib /*32 nibble values*/, uint8_t* scale_byte);
void quant_w8_row(const float* x, int32_t K, int8_t* q, float* scale);

void parallel_for(int64_t n, int threads, const std::function<void(int64_t, int64_t)>& fn);
int default_threads(int requested);

bool top_eigenpairs(double* G, int64_t n, int64_t r, int threads, int max_iters,
                    std::vector<double>& evals, std::vector<double>& evecs);
bool truncated_svd(const double* A, int64_t K, int64_t N, int64_t r, int threads, int max_iters,
                   std::vector<double>& L1, std::vector<double>& L2, std::vector<double>& sigma);

}  // namespace svdq
