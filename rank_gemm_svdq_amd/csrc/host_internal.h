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
inline bool is_mx(int fmt) { return fmt == SVDQ_MXFP4_G32 || fmt == SVDQ_MXFP4_G32_OCP; }   // same layouts
// code steps of 64 bytes per row: 128 elements (4-bit) or 64 (8-bit)
inline int32_t code_steps(int32_t K, int fmt) { return is_w8(fmt) ? K / 64 : K / 128; }
// canonical buffers: codes [rows, K/2] (4-bit) or [rows, K] (8-bit); scales
// [rows, K/64] fp16, [rows, K/32] E8M0 or [rows] fp32
inline size_t canon_code_bytes(int64_t rows, int32_t K, int fmt) {
  return is_w8(fmt) ? (size_t)rows * K : (size_t)rows * (K / 2);
}
inline size_t canon_scale_bytes(int64_t rows, int32_t K, int fmt) {
  return fmt == SVDQ_INT4_G64 ? (size_t)rows * (K / 64) * 2 : is_mx(fmt) ? (size_t)rows * (K / 32)
                                                                                   : (size_t)rows * 4;
}
inline int32_t rank_pad(int32_t rank) { return (rank + 31) / 32 * 32; }
inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Kernel-layout geometry (documented in the device source and DESIGN notes)
struct Geometry {
  int32_t K, N, rank, rpad, fmt, steps, ks4, csteps;   // csteps: 64-byte code steps per row
  size_t wq_bytes, ws_bytes, l1k_bytes, l2k_bytes;
  size_t wq_tail_off;                                  // INT4: start of the code tails inside wq
};
bool geometry(int32_t K, int32_t N, int32_t rank, int32_t fmt, Geometry* g);
bool valid_kn(int32_t K, int32_t N);
bool valid_rank(int32_t rank);
bool valid_fmt(int32_t fmt);
int32_t choose_zsplit(int32_t M, int32_t K);

// INT4 codes on the device: 32 six-bit FP6 codes of a slice packed into 6
// dwords, element j at bits 6 j, and back.
inline void pack6(const uint8_t* c32, uint32_t* d6) {
  for (int i = 0; i < 6; ++i) d6[i] = 0;
  for (int j = 0; j < 32; ++j) {
    const int bit = 6 * j;
    const uint64_t v = (uint64_t)(c32[j] & 63) << (bit & 31);
    d6[bit >> 5] |= (uint32_t)v;
    if ((bit & 31) + 6 > 32) d6[(bit >> 5) + 1] |= (uint32_t)(v >> 32);
  }
}
inline void unpack6(const uint32_t* d6, uint8_t* c32) {
  for (int j = 0; j < 32; ++j) {
    const int bit = 6 * j;
    uint64_t v = d6[bit >> 5] >> (bit & 31);
    if ((bit & 31) + 6 > 32) v |= (uint64_t)d6[(bit >> 5) + 1] << (32 - (bit & 31));
    c32[j] = (uint8_t)(v & 63);
  }
}
// INT4 value of an FP6 E2M3 code the packers write; 8 (an INT4 nibble the
// quantizers never produce) for any other code.
struct E2m3Inverse {
  int8_t q[64];
  E2m3Inverse() {
    for (int c = 0; c < 64; ++c) q[c] = c == 0x20 ? 0 : 8;
    for (int v = -7; v <= 7; ++v) q[e2m3_of_int4(v)] = (int8_t)v;
  }
};
inline int int4_of_e2m3(uint8_t c) {
  static const E2m3Inverse inv;
  return inv.q[c & 63];
}

// Scalar conversions (round to nearest even).
uint16_t bf16_from_double(double x);
double double_from_bf16(uint16_t h);
uint16_t half_from_float(float x);
float float_from_half(uint16_t h);

// Quantizers of one group, shared by the weight packer and the unpack helper.
void quant_int4_group(const float* x, uint8_t* nib /*64 nibble values*/, uint16_t* scale_bits);
void quant_mxfp4_group(const float* x, uint8_t* nib /*32 nibble values*/, uint8_t* scale_byte, bool ocp_rule);
void quant_w8_row(const float* x, int32_t K, int8_t* q, float* scale);

// One residual-iteration candidate as a deployable layer (canonical host
// buffers, valid during the call), and a function that scores it in place
// of the weight reconstruction error (the smooth search's calibration
// output error).
struct CandidateView {
  const float* lambda;
  const float* smooth_inv;
  const uint16_t* l1b;   // [K, rank] (NULL when rank == 0)
  const uint16_t* l2b;   // [rank, N]
  const uint8_t* wq;     // canonical codes
  const uint8_t* ws;     // canonical scales
};
using Scorer = std::function<svdq_status(const CandidateView&, double* score)>;

// svdq_prepare with an optional scorer of the residual iterations.
svdq_status prepare_layer(const float* W, const float* act_amax, int32_t K, int32_t N, double alpha, int32_t rank,
                          int32_t fmt, const svdq_prepare_opts* opts, svdq_prepared* out, const Scorer* scorer);

void parallel_for(int64_t n, int threads, const std::function<void(int64_t, int64_t)>& fn);
int default_threads(int requested);

bool top_eigenpairs(double* G, int64_t n, int64_t r, int threads, int max_iters,
                    std::vector<double>& evals, std::vector<double>& evecs);
bool truncated_svd(const double* A, int64_t K, int64_t N, int64_t r, int threads, int max_iters,
                   std::vector<double>& L1, std::vector<double>& L2, std::vector<double>& sigma);

}  // namespace svdq
