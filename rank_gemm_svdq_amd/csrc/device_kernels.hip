// gfx950 kernels of the SVDQuant W4A4 + low-rank linear layer and the device
// entry points of the C ABI.
//
// Dataflow (Zhou, SVDQuant reading notes, sec. 6.1, Algorithm 2): K-A reads a
// tile of X once and produces both the 4-bit activation codes/scales and the
// down projection Z = X^ L1'; K-B runs the 4-bit main contraction and merges
// Z L2' and the bias into the same fp32 accumulators before the single bf16
// store of Y.
//
// MFMA operand conventions (checked on the device by lane-layout probes):
// for v_mfma_*_16x16x{32 bf16, 64 i8, 128 f4}, lane l supplies row l % 16 of
// A (and column l % 16 of B) for the K slice owned by lane group l / 16; the
// K slices of A and B pair up by lane group.  The 16x16 fp32 result lives in
// lane l, register i at row 4 (l / 16) + i, column l % 16.  The scaled FP4
// MFMA applies lane l's E8M0 byte to the 32 values lane l supplies.
//
// K-B computes Y^T tiles: A = weights (rows n), B = activations (rows m), so
// each lane owns 4 consecutive outputs n of one token m (an 8-byte store).
//
// Layouts (offsets in layout.h; K split into steps of 64 code bytes per
// row: 128 4-bit elements or 64 int8 elements):
//   Codes (activations and weights, every format): 1 KB units of 16 rows x
//     one step, ordered [row / 16][step]; inside a unit, 16-byte slot
//     4 (row % 16) + q holds chunk q ^ swz(row % 32) of the row-step.  MXFP4
//     and W8A8 keep canonical byte order inside a row-step; INT4 places
//     element k (G = k / 64, g = k % 64 / 16, j = k % 16) at byte
//     16 g + 8 G + j / 2, nibble j % 2, so the 16 bytes of lane group g
//     hold 16 elements of each of the step's two 64-element groups.
//   Scale records (MXFP4 both operands, INT4 activations): 1 KB units of 64
//     rows x 4 steps ordered [row / 64][4-step group]; dword d of row r sits
//     at unit dword 64 (r % 64 / 16) + 16 d + r % 16.  MXFP4: dword d holds
//     the E8M0 scales of 32-element block d of the 4 steps (byte t % 4), the
//     weight rows permuted inside their 64-row group (wrec_row); INT4: dword
//     t % 4 is the fp16 pair of step t.
//   INT4 weight scales: 2 KB units of 128 rows x 4 steps, [4-row block]
//     [step % 4][row % 4][group of 64] fp16.
//   W8A8 scales: fp32 per token row (workspace) and per out-feature (layer).
//   Down factor: L1' (bf16), ordered [step][s][n-tile < rank/16][lane][8]
//     with k = 128 step + 32 (lane/16) + 8 s + i, n = 16 n-tile + lane % 16.
//   Up factor: L2'^T, [N][rpad] bf16, rpad = rank rounded up to 32.
//   Z (down projection): per row and 32-column chunk, 32 bf16 hi values then
//     32 bf16 lo values (hi + lo = Z to about 2^-17), rpad * 4 bytes per row.

#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>
#include <cstdint>
#include <cstring>

#include "host_internal.h"

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ----------------------------------------------------------------- K-A

constexpr int KA_WAVES = 8;
constexpr int KA_SL_MAX_K = 16384;   // 1/lambda is staged in LDS up to this K

// One block handles 16 rows; its 8 waves split the K steps evenly and the
// down-projection partial sums are reduced in LDS, so Z leaves the kernel
// once.  Lane l owns row l % 16 and the 32 consecutive elements
// 32 (l / 16) .. +32 of each 128-element step.  Each wave keeps the next
// two steps' X (and, for ranks up to 64, their down-factor fragments) in
// flight in a register ring while it processes the current one; 1/lambda
// comes from LDS when K allows.  The down projection multiplies the
// smoothed x^ = x / lambda, split into bf16 hi + lo, by the bf16 factor
// L1', so it runs on bf16 MFMA with fp32 accumulation.  ZONLY drops the
// quantisation (the unfused baseline's separate down-projection pass).
template <int FMT, int NT, bool SL, bool ZONLY = false, bool RING = true>
__global__ __launch_bounds__(64 * KA_WAVES) void ka_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                          const float* __restrict__ sinv,
                                                          const v8bf* __restrict__ l1k,
                                                          uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                                          float* __restrict__ zout, int rpad) {
  constexpr int NTZ = NT > 0 ? NT : 1;
  // down-factor fragments in the ring (RING: chosen when one block per
  // compute unit runs; without them the kernel fits two blocks per unit)
  constexpr bool WRING = RING && NT > 0 && NT <= (SL ? 4 : 2);
  constexpr int NW = WRING ? 4 * NT : 1;
  constexpr bool W8 = FMT == SVDQ_W8A8 && !ZONLY;
  __shared__ float zred[NT > 0 ? KA_WAVES * 16 * NT * 16 : 1];
  __shared__ float mred[W8 ? KA_WAVES * 16 : 1];
  extern __shared__ __attribute__((aligned(16))) float svl[];   // K floats when SL
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * 16;
  const int r = lane & 15, g = lane >> 4;
  const int row = row0 + r;
  const int rowc = row < M ? row : M - 1;
  const bool live = row < M;
  const int steps = K / 128;
  const int ks4 = (steps + 3) / 4;
  const int spw = (steps + KA_WAVES - 1) / KA_WAVES;
  const int t0 = wave * spw;
  const int t1 = min(steps, t0 + spw);
  const uint16_t* xrow = X + (size_t)rowc * K + 32 * g;

  struct Slot {
    v4i x[4];
    v4f s[SL ? 1 : 8];
    v8bf w[NW];
  };
  auto load = [&](int t, Slot& sl) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) sl.x[c] = *reinterpret_cast<const v4i*>(xrow + (size_t)t * 128 + 8 * c);
    if constexpr (!SL) {
#pragma unroll
      for (int c = 0; c < 8; ++c) sl.s[c] = *reinterpret_cast<const v4f*>(sinv + t * 128 + 32 * g + 4 * c);
    }
    if constexpr (WRING) {
#pragma unroll
      for (int i = 0; i < 4 * NT; ++i) sl.w[i] = l1k[((size_t)t * 4 * NT + i) * 64 + lane];
    }
  };
  if constexpr (SL) {
    for (int i = 4 * (int)threadIdx.x; i < K; i += 4 * 64 * KA_WAVES)
      *reinterpret_cast<v4f*>(svl + i) = *reinterpret_cast<const v4f*>(sinv + i);
  }
  Slot ring[2];
  if (t0 < t1) load(t0, ring[0]);
  if (t0 + 1 < t1) load(t0 + 1, ring[1]);
  if constexpr (SL) __syncthreads();

  v4f acc[NTZ];
#pragma unroll
  for (int nt = 0; nt < NTZ; ++nt) acc[nt] = (v4f){0.f, 0.f, 0.f, 0.f};
  float rmax = 0.f;   // W8A8: running |x^| maximum of this lane's share of its row

  // x^ = fp32(x * 1/lambda) for the lane's 32 elements of step t
  auto smooth = [&](int t, const Slot& sl, float* xh) __attribute__((always_inline)) {
    const int k0 = t * 128 + 32 * g;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const v4f iv = SL ? *reinterpret_cast<const v4f*>(svl + k0 + 4 * c) : sl.s[SL ? 0 : c];
      const uint32_t w0 = (uint32_t)sl.x[c >> 1][(c & 1) * 2], w1 = (uint32_t)sl.x[c >> 1][(c & 1) * 2 + 1];
      xh[4 * c + 0] = bf16_lo(w0) * iv[0];
      xh[4 * c + 1] = bf16_hi(w0) * iv[1];
      xh[4 * c + 2] = bf16_lo(w1) * iv[2];
      xh[4 * c + 3] = bf16_hi(w1) * iv[3];
    }
  };

  auto process = [&](int t, const Slot& sl) __attribute__((always_inline)) {
    float xh[32];
    smooth(t, sl, xh);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(xh[i]));

    if constexpr (ZONLY) {
      // down projection only (the unfused baseline's separate pass over X)
    } else if constexpr (FMT == SVDQ_W8A8) {
      // per-token scale: the whole row's maximum is needed first; the codes
      // are written in a second pass below
      rmax = fmaxf(rmax, amax);
    } else if constexpr (FMT == SVDQ_MXFP4_G32) {
      // smallest e with amax <= 6 * 2^e, clamped to [-127, 127]
      const uint32_t ab = __float_as_uint(amax);
      const int ex = (int)(ab >> 23);
      int e = ex == 0 ? -127 : ex - 129 + ((ab & 0x7FFFFFu) > 0x400000u ? 1 : 0);
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
      v4i packed;
      if (e >= -126) {
        const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t d = 0;
          d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, xh[8 * w + 0], xh[8 * w + 1], scale, 0);
          d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, xh[8 * w + 2], xh[8 * w + 3], scale, 1);
          d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, xh[8 * w + 4], xh[8 * w + 5], scale, 2);
          d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, xh[8 * w + 6], xh[8 * w + 7], scale, 3);
          packed[w] = (int)d;
        }
      } else {
        // block maximum below 6 * 2^-126: exact comparison against the E2M1
        // midpoints of |x| * 2^127 (no denormal scale operand)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t d = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float v = xh[8 * w + j];
            const float a = fabsf(v) * 1.7014118346046923e38f;   // 2^127
            uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
                         (a > 5.0f);
            c |= (__float_as_uint(v) >> 28) & 8u;
            d |= c << (4 * j);
          }
          packed[w] = (int)d;
        }
      }
      if (live) {
        *reinterpret_cast<v4i*>(xq + code_offset(row, t, 16 * g, steps)) = packed;
        xs[scale_record_offset(row, t >> 2, 4 * g + (t & 3), ks4)] = (uint8_t)(e + 127);
      }
    } else {
      // INT4: the 64-element group spans lane groups g and g ^ 1
      const float amax64 = fmaxf(amax, __shfl_xor(amax, 16));
      const float s32 = amax64 / 7.0f;
      const _Float16 s16 = (_Float16)s32;
      const float sf = (float)s16;
      uint32_t d[4] = {0u, 0u, 0u, 0u};
      if (sf != 0.f) {
        const float rcp = 1.0f / sf;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          float q = __builtin_rintf(xh[i] * rcp);
          q = fminf(fmaxf(q, -7.f), 7.f);
          d[i >> 3] |= ((uint32_t)(int)q & 0xFu) << (4 * (i & 7));
        }
      }
      if (live) {
        // bytes 32 half + 8 G + (0..7) and the same + 16 of the step (the
        // INT4 step permutation), each inside one 16-byte chunk
        const int G = g >> 1, half = g & 1;
        *reinterpret_cast<uint2*>(xq + code_offset(row, t, 32 * half + 8 * G, steps)) = make_uint2(d[0], d[1]);
        *reinterpret_cast<uint2*>(xq + code_offset(row, t, 32 * half + 16 + 8 * G, steps)) = make_uint2(d[2], d[3]);
        if (half == 0) {
          uint16_t sb;
          __builtin_memcpy(&sb, &s16, 2);
          *reinterpret_cast<uint16_t*>(xs + scale_record_offset(row, t >> 2, 4 * (t & 3) + 2 * G, ks4)) = sb;
        }
      }
    }

    if constexpr (NT > 0) {
      // Z += (x^hi + x^lo) L1': MFMA s covers elements 32 g + 8 s .. + 8 of
      // every lane group, i.e. k = 128 t + 32 (lane / 16) + 8 s + i.
      // hi = bf16_rne(x^) and lo = bf16_rne(x^ - hi) (the difference is
      // exact in fp32), both converted two elements at a time; hi is widened
      // back from its packed bits by a shift or a mask
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        v4i hw, lw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = xh[8 * s4 + 2 * i], x1 = xh[8 * s4 + 2 * i + 1];
          const uint32_t hp = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){x0, x1}, v2bf));
          const float r0 = x0 - __uint_as_float(hp << 16), r1 = x1 - __uint_as_float(hp & 0xFFFF0000u);
          hw[i] = (int)hp;
          lw[i] = (int)__builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){r0, r1}, v2bf));
        }
        const v8bf hi = __builtin_bit_cast(v8bf, hw), lo = __builtin_bit_cast(v8bf, lw);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const v8bf b = WRING ? sl.w[WRING ? s4 * NT + nt : 0] : l1k[(((size_t)t * 4 + s4) * NT + nt) * 64 + lane];
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc[nt], 0, 0, 0);
        }
      }
    }
  };

  for (int t = t0; t < t1; t += 2) {
    process(t, ring[0]);
    if (t + 2 < t1) load(t + 2, ring[0]);
    if (t + 1 < t1) {
      process(t + 1, ring[1]);
      if (t + 3 < t1) load(t + 3, ring[1]);
    }
  }
  if constexpr (NT > 0) {
    // partial sums of wave w: rows 4 g + i, columns 16 nt + r
    constexpr int W = NT * 16;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) zred[(wave * 16 + 4 * g + i) * W + 16 * nt + r] = acc[nt][i];
    __syncthreads();
    // columns from the rank up to WP = rpad (the rank rounded up to 32) are
    // written as 0
    constexpr int WP = (W + 31) / 32 * 32;
    for (int idx = threadIdx.x; idx < 16 * WP; idx += 64 * KA_WAVES) {
      const int rr = idx / WP, cc = idx % WP;
      float sum = 0.f;
      if (cc < W) {
#pragma unroll
        for (int w = 0; w < KA_WAVES; ++w) sum += zred[(w * 16 + rr) * W + cc];
      }
      // Z leaves as the bf16 pair hi + lo the up projection multiplies with:
      // per row and 32-column chunk, 32 hi values then 32 lo values
      if (row0 + rr < M) {
        const __bf16 hi = (__bf16)sum;
        const __bf16 lo = (__bf16)(sum - (float)hi);
        uint16_t* zr = reinterpret_cast<uint16_t*>(zout) + (size_t)(row0 + rr) * 2 * WP + 64 * (cc >> 5) + (cc & 31);
        zr[0] = __builtin_bit_cast(uint16_t, hi);
        zr[32] = __builtin_bit_cast(uint16_t, lo);
      }
    }
  }
  if constexpr (W8) {
    // row maximum over the 4 lane groups and the 8 waves, then s = amax/127
    // and a second pass over the wave's steps (X is re-read, now from cache)
    float m = fmaxf(rmax, __shfl_xor(rmax, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (g == 0) mred[wave * 16 + r] = m;
    __syncthreads();
    float am = 0.f;
#pragma unroll
    for (int w = 0; w < KA_WAVES; ++w) am = fmaxf(am, mred[w * 16 + r]);
    const float sc = am / 127.0f;
    if (wave == 0 && g == 0 && live) reinterpret_cast<float*>(xs)[row] = sc;
    const float rcp = 1.0f / sc;   // sc == 0 only for an all-zero row
    const int steps8 = 2 * steps;
    for (int t = t0; t < t1; ++t) {
      Slot sl;
#pragma unroll
      for (int c = 0; c < 4; ++c) sl.x[c] = *reinterpret_cast<const v4i*>(xrow + (size_t)t * 128 + 8 * c);
      if constexpr (!SL) {
#pragma unroll
        for (int c = 0; c < 8; ++c) sl.s[c] = *reinterpret_cast<const v4f*>(sinv + t * 128 + 32 * g + 4 * c);
      }
      float xh[32];
      smooth(t, sl, xh);
      uint32_t d[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        d[w] = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // a zero stays 0 also when rcp is infinite (s below 2^-128)
          float q = xh[4 * w + j] == 0.f ? 0.f : __builtin_rintf(xh[4 * w + j] * rcp);
          q = fminf(fmaxf(q, -127.f), 127.f);
          d[w] |= ((uint32_t)(int)q & 0xFFu) << (8 * j);
        }
      }
      if (live) {
        // elements 128 t + 32 g .. +32: bytes 32 (g & 1) .. +32 of 8-bit step 2 t + g / 2
        const int t8 = 2 * t + (g >> 1), b0 = 32 * (g & 1);
        *reinterpret_cast<v4i*>(xq + code_offset(row, t8, b0, steps8)) =
            (v4i){(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
        *reinterpret_cast<v4i*>(xq + code_offset(row, t8, b0 + 16, steps8)) =
            (v4i){(int)d[4], (int)d[5], (int)d[6], (int)d[7]};
      }
    }
  }
}

// ----------------------------------------------------------------- K-B

// swizzled byte offset of 16-byte chunk c of row r inside a [rows][64 B]
// tile: the codes layout's XOR swizzle (chunk_swz, which makes the fragment
// reads free of LDS bank conflicts)
__device__ __forceinline__ int swz(int r, int c) { return r * 64 + 16 * (c ^ chunk_swz(r)); }

// ----------------------------------------------------- K-B, MXFP4, large tile
//
// 256 (tokens) x 256 (out-features) per block of 8 waves, two per SIMD; wave
// w owns tokens 128 (w & 1) .. +128 and out-features 64 (w >> 1) .. +64, i.e.
// 4 x 8 MFMA tiles of 16 x 16 (128 fp32 accumulators per lane).
//
// Codes travel global -> LDS by direct-to-LDS loads (no register staging)
// into a ring of four 32 KB step buffers; scale dwords (one per row and 4
// steps) travel the same way into a double buffer.  The K loop runs in
// pairs of steps with one barrier per pair: the first step of a pair loads
// the next pair into the two buffers the previous pair has left.  The
// weight fragments of the next step are read into the other half of a
// two-deep register set while the current MFMAs run, and token fragments
// stream through four registers three MFMA groups ahead, so no fragment is
// ever copied between registers.  A 16-bit LDS read per pair gives each
// scale register the E8M0 bytes of both steps; the MFMA's op_sel picks the
// byte.  The low-rank product Z L2' is formed before the K loop while the
// first code steps are in flight (MXFP4), or after it from Z and L2' tiles
// loaded into ring buffers the last pair no longer uses (W8A8).
//
// Weight rows are permuted inside each pair of 16-row MFMA tiles (2p, 2p+1):
// MFMA row q of tile 2p + h is out-feature 32 p + 8 (q / 4) + 4 h + q % 4, so
// the 4 + 4 accumulators a lane holds for the pair are 8 consecutive
// out-features of one token: one 16-byte store.

constexpr int MX_BM = 256, MX_BN = 256;
#ifndef SVDQ_MX_WAVES
#define SVDQ_MX_WAVES 8
#endif
constexpr int MX_STEP_BYTES = (MX_BM + MX_BN) * 64;   // codes of one step, both operands
constexpr int MX_NBUF = 4;
constexpr int MX_SC_BYTES = (MX_BM + MX_BN) * 16;     // scale dwords of one 4-step group
constexpr int MX_DUMMY = MX_NBUF * MX_STEP_BYTES + 2 * MX_SC_BYTES;   // 1 KB per wave, see below
constexpr int MX_LDS = MX_DUMMY + 8 * 1024;
constexpr int MX_LDS_LRF = MX_DUMMY + 16 * 1024;   // the dummy region doubles as the first L2' chunk

#define SVDQ_AS3 __attribute__((address_space(3)))

// One wave-wide 1 KB direct-to-LDS copy: lane i's 16 bytes at sbase + voff
// (sbase wave-uniform, voff per lane) land at LDS byte lds_base + 16 i.
// Issued from asm so that the compiler does not serialise it against
// unrelated LDS reads; completion is tracked with explicit vmcnt waits.
// M0 is restored before the asm block ends.
__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(sbase)
      : "memory");
}

// Blocks are dealt to the 8 XCDs round robin; give each XCD a contiguous run
// of tile ids (a band of out-feature tiles, all token tiles), and order the
// run in groups of 8 token tiles, out-feature tile slower, so the ~32 blocks
// resident on one XCD at a time cover about 8 token x 4 out-feature tiles:
// 12 operand panels share its L2 instead of 16 + 2.
__device__ __forceinline__ void mx_tile_of(int b, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int total = tiles_m * tiles_n;
  int id = b;
  if (total % 8 == 0) id = (b & 7) * (total / 8) + (b >> 3);
  const int gm = 8;
  const int full = tiles_m / gm * gm;             // token tiles in whole groups
  const int span = gm * tiles_n;                  // ids per whole group
  if (id < full * tiles_n) {
    const int grp = id / span, r = id % span;
    *tm = grp * gm + r % gm;
    *tn = r / gm;
  } else {                                        // the last, partial group
    const int r = id - full * tiles_n, rem = tiles_m - full;
    *tm = full + r % rem;
    *tn = r / rem;
  }
}

// LDS swizzles of the low-rank tiles read in the epilogues: Z rows are
// 128 bytes (8 chunks of 16), L2'^T rows 64 bytes (4 chunks); chunk c of row
// r sits at chunk position c ^ f(r), so the 8 lanes served together by a
// 16-byte LDS read (consecutive, or pair-permuted, rows) hit 8 distinct
// 16-byte slots of a 128-byte line.
__device__ __forceinline__ int zswz(int r) { return r & 7; }
__device__ __forceinline__ int lswz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// out-feature (relative to the wave's 64) of MFMA row q of weight tile nt
__device__ __forceinline__ int mx_nrow(int nt, int q) {
  return 32 * (nt >> 1) + 8 * (q >> 2) + 4 * (nt & 1) + (q & 3);
}

template <int NTR, bool ODD, int WAVES, bool W8 = false>
__global__ __launch_bounds__(WAVES * 64, 1) void kb_mx_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const float* __restrict__ zp,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const uint16_t* __restrict__ l2k,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int N, int K, int rpad) {
  // LRF: the low-rank product Z L2' is formed first, while the first code
  // steps are in flight (float accumulators only, so not for W8)
  constexpr bool LRF = !W8 && NTR > 0;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LRF ? MX_LDS_LRF : MX_LDS];
  const uint32_t lds_u32 = (uint32_t)(size_t)(SVDQ_AS3 uint8_t*)lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // WAVES = 8: waves own 128 tokens x 64 out-features; WAVES = 4: 128 x 128
  constexpr int NTW = 32 / WAVES;        // 16-row weight tiles per wave
  constexpr int UPW = 32 / WAVES;        // 1 KB code units per wave and step
  constexpr int RPW = 8 / WAVES;         // 1 KB scale records per wave and 4 steps
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g = lane >> 4;
  const int tiles_m = (M + MX_BM - 1) / MX_BM, tiles_n = (N + MX_BN - 1) / MX_BN;
  int tm, tn;
  mx_tile_of(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int tile_m = tm * MX_BM, tile_n = tn * MX_BN;
  // 64-byte code steps: 128 FP4 elements, or 64 int8 elements (W8)
  const int steps = W8 ? K / 64 : K / 128;
  const int ks4 = (steps + 3) / 4;
  const int m_base = tile_m + 128 * wm, n_base = tile_n + 16 * NTW * wn;

  // ---- DMA plan.  Codes are stored in 1 KB units of 16 rows x one step, in
  // the order the step buffers hold them (codes layout), so every load is
  // one contiguous kilobyte: wave w moves units UPW w .. UPW w + UPW - 1 of
  // a step buffer (units 0-15: token rows, 16-31: weight rows), lane i 16
  // bytes.  Units past the last row group repeat it (their outputs are
  // never stored).  Lane offsets are 32-bit (operands below 2 GiB, checked
  // on the host).
  const bool tokw = wave < WAVES / 2;
  const uint8_t* cbase = tokw ? xq : wq;
  const int gmax = tokw ? (M + 15) / 16 - 1 : N / 16 - 1;
  const int g0 = (tokw ? tile_m : tile_n) >> 4;
  uint32_t coff[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int grp16 = min(g0 + ((UPW * wave + j) & 15), gmax);
    coff[j] = (uint32_t)grp16 * (uint32_t)steps * 1024u + 16u * lane;
  }
  // Scales: 1 KB records of 64 rows x 4 steps, 8 per 4-step group (records
  // 0-3 token rows, 4-7 weight rows); wave w moves records RPW w ..
  const uint8_t* sbase = tokw ? xs : ws;
  const int smax = tokw ? (M + 63) / 64 - 1 : (N + 63) / 64 - 1;
  uint32_t soff[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int grp64 = min(((tokw ? tile_m : tile_n) >> 6) + ((RPW * wave + j) & 3), smax);
    soff[j] = (uint32_t)grp64 * (uint32_t)ks4 * 1024u + 16u * lane;
  }
  const uint32_t scale_lds = lds_u32 + MX_NBUF * MX_STEP_BYTES;
  auto issue_codes = [&](int t) __attribute__((always_inline)) {
    const uint32_t b = lds_u32 + (uint32_t)(t % MX_NBUF) * MX_STEP_BYTES + (uint32_t)wave * (1024u * UPW);
#pragma unroll
    for (int j = 0; j < UPW; ++j) dma16(cbase + (size_t)t * 1024, coff[j], b + 1024u * j);
  };
  auto issue_scales = [&](int grp) __attribute__((always_inline)) {
    if constexpr (W8) return;   // W8: per-row scales, applied after the K loop
#pragma unroll
    for (int j = 0; j < RPW; ++j)
      dma16(sbase + (size_t)grp * 1024, soff[j],
            scale_lds + (uint32_t)(grp & 1) * MX_SC_BYTES + (uint32_t)(RPW * wave + j) * 1024u);
  };

  // fragment addresses (without the step-buffer offset): token fragment q
  // reads row 128 wm + 16 q + l16 (two parities, 1 KB apart per q), weight
  // fragment nt reads the permuted row 16 NTW wn + mx_nrow(nt, l16)
  uint32_t boff[2], aoff[NTW];
#pragma unroll
  for (int par = 0; par < 2; ++par) boff[par] = (uint32_t)swz(128 * wm + 16 * par + l16, g) - 1024u * par;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) aoff[nt] = (uint32_t)(MX_BM * 64 + swz(16 * NTW * wn + mx_nrow(nt, l16), g));
  // bo: byte offset of a step buffer, kept opaque to the optimiser so that
  // it does not hoist one address register per (buffer, fragment) pair out
  // of the unrolled loop
  auto buf_of = [&](int t) __attribute__((always_inline)) -> uint32_t {
    uint32_t bo = (uint32_t)(t % MX_NBUF) * MX_STEP_BYTES;
    asm volatile("" : "+s"(bo));
    return bo;
  };
  auto read_b = [&](uint32_t bo, int q) __attribute__((always_inline)) -> v4i {
    return *reinterpret_cast<const v4i*>(lds + bo + boff[q & 1] + 1024 * q);
  };
  auto read_a = [&](uint32_t bo, int nt) __attribute__((always_inline)) -> v4i {
    return *reinterpret_cast<const v4i*>(lds + bo + aoff[nt]);
  };
  // Scale registers: the lane's record dword holds the E8M0 bytes of the 4
  // steps of a group; it is read at the group's first pair (tp % 4 == 0)
  // and shifted down by 16 bits for its second, so that the bytes of steps
  // (tp, tp+1) always sit in the low half and the MFMA's op_sel picks byte J.
  uint32_t asc[NTW], bsc[8];
  auto read_scales = [&](int tp) __attribute__((always_inline)) {
    if constexpr (W8) return;
    if ((tp & 3) != 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) bsc[q] >>= 16;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) asc[nt] >>= 16;
      return;
    }
    uint32_t so = (uint32_t)(MX_NBUF * MX_STEP_BYTES + ((tp >> 2) & 1) * MX_SC_BYTES);
    asm volatile("" : "+s"(so));
    const uint8_t* sc = lds + so;
    // 1 KB records of 64 rows: token fragment q is rows 16 (q % 4) .. of
    // record 2 wm + q / 4; the weight records hold the wave's fragments in
    // order (16 rows per tile nt); dword g of 16 rows = 256 contiguous bytes
#pragma unroll
    for (int q = 0; q < 8; ++q)
      bsc[q] = *reinterpret_cast<const uint32_t*>(sc + 1024 * (2 * wm + (q >> 2)) + 4 * (64 * (q & 3) + 16 * g + l16));
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      asc[nt] = *reinterpret_cast<const uint32_t*>(sc + 1024 * ((MX_BM + 16 * NTW * wn) / 64 + (nt >> 2)) +
                                                   4 * (64 * (nt & 3) + 16 * g + l16));
  };
  // The lane index is made opaque in these two so that their address
  // arithmetic is redone where they are called instead of being hoisted out
  // of the main loop into live registers.
  auto issue_z = [&](int u, uint32_t zdst) __attribute__((always_inline)) {
    // Z: 32 units of 8 rows x 128 B; wave w moves units 32/WAVES each
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j < 32 / WAVES; ++j) {
      const int unit = (32 / WAVES) * wave + j, row = 8 * unit + (ln >> 3);
      const int m = min(tile_m + row, M - 1);
      dma16(reinterpret_cast<const uint8_t*>(zp),
            ((uint32_t)m * (uint32_t)rpad + 32u * u) * 4u + 16u * ((ln & 7) ^ zswz(row)), zdst + 1024u * unit);
    }
  };
  auto issue_l2 = [&](int u, uint32_t ldst) __attribute__((always_inline)) {
    // L2'^T: 16 units of 16 rows x 64 B; wave w moves units 16/WAVES each
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j < 16 / WAVES; ++j) {
      const int unit = (16 / WAVES) * wave + j, row = 16 * unit + (ln >> 2);
      const int n = min(tile_n + row, N - 1);
      dma16(reinterpret_cast<const uint8_t*>(l2k),
            ((uint32_t)n * (uint32_t)rpad + 32u * u) * 2u + 16u * ((ln & 3) ^ lswz(row)), ldst + 1024u * unit);
    }
  };
  // acc += Z L2' for one 32-column chunk of the rank, from Z (rows of the
  // wave's tokens, bf16 hi and lo) and L2'^T (rows of its out-features) in LDS
  auto lr_mfma = [&](uint32_t zoff, uint32_t loff, v4f (&ac)[NTW][8]) __attribute__((always_inline)) {
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
      v8bf bh[4], bl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int mt = 4 * mh + k;
        const int zrow = 128 * wm + 16 * mt + l16;
        bh[k] = *reinterpret_cast<const v8bf*>(lds + zoff + zrow * 128 + 16 * (g ^ zswz(zrow)));
        bl[k] = *reinterpret_cast<const v8bf*>(lds + zoff + zrow * 128 + 16 * ((4 + g) ^ zswz(zrow)));
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int lrow = 16 * NTW * wn + mx_nrow(nt, l16);
        const v8bf af = *reinterpret_cast<const v8bf*>(lds + loff + lrow * 64 + 16 * (g ^ lswz(lrow)));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ac[nt][4 * mh + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh[k], ac[nt][4 * mh + k], 0, 0, 0);
          ac[nt][4 * mh + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl[k], ac[nt][4 * mh + k], 0, 0, 0);
        }
      }
    }
  };

  v4f acc[NTW][8];   // [weight tile][token tile]
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = (v4f){0.f, 0.f, 0.f, 0.f};

  // Prologue.  LRF: chunk 0 of Z goes to ring buffer 3 and of L2' to the
  // dummy region (neither is written by code loads before step 0 has passed
  // its barrier), ahead of the scales and code steps 0-1; the low-rank MFMAs
  // run as soon as those two have landed, while the code steps are still in
  // flight.
  constexpr uint32_t LR_Z = 3 * MX_STEP_BYTES, LR_L = MX_DUMMY;
  if constexpr (LRF) {
    issue_z(0, lds_u32 + LR_Z);
    issue_l2(0, lds_u32 + LR_L);
  }
  issue_scales(0);
#pragma unroll
  for (int s0 = 0; s0 < 2; ++s0)
    if (s0 < steps) issue_codes(s0);
  if constexpr (LRF) {
    for (int u = 0; u < NTR; ++u) {
      if (u == 0) {
        // everything issued after the Z / L2' loads may still be in flight
        if (steps >= 2) {
          if constexpr (WAVES == 8)
            asm volatile("s_waitcnt vmcnt(9)" ::: "memory");    // 1 scale record + 2 x 4 code units
          else
            asm volatile("s_waitcnt vmcnt(18)" ::: "memory");   // 2 + 2 x 8
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
      } else {
        __syncthreads();   // every wave is done with chunk u-1
        issue_z(u, lds_u32 + LR_Z);
        issue_l2(u, lds_u32 + LR_L);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
      lr_mfma(LR_Z, LR_L, acc);
    }
  }

  v4i wf[2][NTW];   // weight fragments of the current and the next step
  v4i tk[4];      // token fragments, three ahead; fragment q sits in slot q & 3

  // The K loop runs in pairs of steps (t, t+1), t even, with one barrier
  // per pair.  At the top of a pair every wave waits for all its loads and
  // passes the barrier: steps t and t+1 are then in LDS, and the two ring
  // buffers of the previous pair are free for steps t+2 and t+3, whose
  // loads the first step of the pair issues (one 1 KB unit per MFMA group
  // with 8 waves).  Loads past the last step re-read it into this wave's
  // dummy region (in bounds, and the loop stays free of branches).
  //
  // Chunk 0 of Z and L2' (the low-rank epilogue, W8) is fetched at the top
  // of the last pair, t_last, into the buffers of t_last-2 and t_last-1,
  // which no load targets any more.
  const int t_last = (steps - 1) & ~1;
  const bool lr_prefetch = !LRF && NTR > 0 && t_last >= 2;
  const uint32_t zpre = (uint32_t)((t_last + 2) % MX_NBUF) * MX_STEP_BYTES;
  const uint32_t lpre = (uint32_t)((t_last + 3) % MX_NBUF) * MX_STEP_BYTES;
  auto pair_top = [&](int t) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if ((t & 3) == 0 && (t >> 2) + 1 < ks4) issue_scales((t >> 2) + 1);
    if (lr_prefetch && t == t_last) {
      issue_z(0, lds_u32 + zpre);
      issue_l2(0, lds_u32 + lpre);
    }
    // scale bytes of steps t, t+1 and the first fragments of step t
    const uint32_t b0 = buf_of(t);
    read_scales(t);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) wf[0][nt] = read_a(b0, nt);
#pragma unroll
    for (int q = 0; q < 3; ++q) tk[q] = read_b(b0, q);
  };
  // step t, J = t & 1.  While the MFMAs of t run, the token fragments three
  // MFMA groups ahead are read and, in the first step of a pair, the weight
  // fragments of t+1.  The scale registers hold the bytes of steps (t & ~1,
  // t | 1) in their low half; the MFMA's op_sel picks byte J.  LAST: the
  // second step of a pair (or a single trailing step), which issues no loads
  // and reads nothing of the next step.
  auto step = [&](int t, auto jtag, auto lasttag) __attribute__((always_inline)) {
    constexpr int J = decltype(jtag)::value;
    constexpr bool LAST = decltype(lasttag)::value;
    const uint32_t bc = buf_of(t), bn = buf_of(t + 1);
    const bool more = t + 2 < steps, more2 = t + 3 < steps;
    const uint8_t* csrc = cbase + (size_t)(more ? t + 2 : steps - 1) * 1024;
    const uint32_t cdst = more ? lds_u32 + (uint32_t)((t + 2) % MX_NBUF) * MX_STEP_BYTES + (uint32_t)wave * (1024u * UPW)
                               : lds_u32 + MX_DUMMY + (uint32_t)wave * 1024u;
    const uint32_t cinc = more ? 1024u : 0u;
    const uint8_t* csrc2 = cbase + (size_t)(more2 ? t + 3 : steps - 1) * 1024;
    const uint32_t cdst2 = more2 ? lds_u32 + (uint32_t)((t + 3) % MX_NBUF) * MX_STEP_BYTES + (uint32_t)wave * (1024u * UPW)
                                 : lds_u32 + MX_DUMMY + (uint32_t)wave * 1024u;
    const uint32_t cinc2 = more2 ? 1024u : 0u;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      if constexpr (!LAST) {
        // groups 0-3 load step t+2, groups 4-7 step t+3; UPW / 4 units each
#pragma unroll
        for (int j = 0; j < UPW / 4; ++j) {
          const int u = (UPW / 4) * (mt & 3) + j;
          if (mt < 4)
            dma16(csrc, coff[u], cdst + cinc * u);
          else
            dma16(csrc2, coff[u], cdst2 + cinc2 * u);
        }
        if (mt < NTW) wf[J ^ 1][mt] = read_a(bn, mt);
        tk[(mt + 3) & 3] = mt + 3 < 8 ? read_b(bc, mt + 3) : read_b(bn, mt - 5);
      } else {
        if (mt + 3 < 8) tk[(mt + 3) & 3] = read_b(bc, mt + 3);
      }
      const v4i bq = tk[mt & 3];
      if constexpr (W8) {
        // int8 x int8 with exact int32 accumulation in the same registers
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          acc[nt][mt] = __builtin_bit_cast(
              v4f, __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[J][nt], bq, __builtin_bit_cast(v4i, acc[nt][mt]), 0, 0, 0));
      } else {
        const v8i b = (v8i){bq[0], bq[1], bq[2], bq[3], 0, 0, 0, 0};
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const v4i aq = wf[J][nt];
          const v8i a = (v8i){aq[0], aq[1], aq[2], aq[3], 0, 0, 0, 0};
          acc[nt][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[nt][mt], 4, 4, J, (int)asc[nt], J,
                                                                        (int)bsc[mt]);
        }
      }
      // keep each group's reads next to its MFMAs: hoisting all reads of a
      // step to its top would need twice the fragment registers
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using L0 = std::integral_constant<bool, false>;
  using L1 = std::integral_constant<bool, true>;
  for (int t0 = 0; t0 < (ODD ? steps - 1 : steps); t0 += 2) {
    pair_top(t0);
    step(t0, J0{}, L0{});
    step(t0 + 1, J1{}, L1{});
  }
  if constexpr (ODD) {
    pair_top(steps - 1);
    step(steps - 1, J0{}, L1{});
  }

  if constexpr (W8) {
    // y = float(I) * (s_w[n] s_x[m]): per-channel weight scale of MFMA row
    // 4 g + i of tile nt, per-token scale of the lane's column
    const float* sxp = reinterpret_cast<const float*>(xs);
    const float* swp = reinterpret_cast<const float*>(ws);
    float sxv[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) sxv[mt] = sxp[min(m_base + 16 * mt + l16, M - 1)];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sw = swp[min(n_base + mx_nrow(nt, 4 * g + i), N - 1)];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
          acc[nt][mt][i] = (float)__builtin_bit_cast(v4i, acc[nt][mt])[i] * (sw * sxv[mt]);
      }
  }
  // ---- low-rank up projection (here only for W8), bias, then one 16-byte
  // store per pair
  if constexpr (NTR > 0 && !LRF) {
    for (int u = 0; u < NTR; ++u) {
      uint32_t zoff, loff;
      if (u == 0 && lr_prefetch) {
        zoff = zpre;
        loff = lpre;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      } else {
        // all ring buffers are idle once every wave has left the main loop
        // (or finished the previous chunk)
        __syncthreads();
        zoff = 0;
        loff = MX_STEP_BYTES;
        issue_z(u, lds_u32 + zoff);
        issue_l2(u, lds_u32 + loff);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
      lr_mfma(zoff, loff, acc);
    }
  }
  // lane holds out-features n_base + 32 p + 8 g + 0..7 of token m for pair p
  auto pack8 = [&](int p2, int mt, const float* bv) __attribute__((always_inline)) -> v4i {
    v4i o;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      o[i] = (int)(bf16_rne(acc[2 * p2][mt][2 * i] + bv[2 * i]) |
                   (bf16_rne(acc[2 * p2][mt][2 * i + 1] + bv[2 * i + 1]) << 16));
      o[2 + i] = (int)(bf16_rne(acc[2 * p2 + 1][mt][2 * i] + bv[4 + 2 * i]) |
                       (bf16_rne(acc[2 * p2 + 1][mt][2 * i + 1] + bv[4 + 2 * i + 1]) << 16));
    }
    return o;
  };
  auto bias8 = [&](int n0, float* bv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) bv[i] = 0.f;
    if (bias != nullptr && n0 < N) {
      const v4i braw = *reinterpret_cast<const v4i*>(bias + n0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bv[2 * i] = bf16_lo((uint32_t)braw[i]);
        bv[2 * i + 1] = bf16_hi((uint32_t)braw[i]);
      }
    }
  };
  if constexpr (NTW == 4 && (NTR > 0 || W8)) {
    // The two pairs cover 128 consecutive bytes of each token row.  Lanes
    // r and r + 8 of a 16-lane row swap one 16-byte piece (DPP row rotate
    // by 8) so that each store instruction writes whole 128-byte lines of
    // 8 rows instead of half lines of 16: HBM writes drop from 1.33x to
    // 1.00x of Y.  (The rank-0 MXFP4 instantiation measured slower with it
    // and keeps the half-line stores.)
    const int n00 = n_base + 8 * g, n01 = n00 + 32;
    float bv0[8], bv1[8];
    bias8(n00, bv0);
    bias8(n01, bv1);
    const bool lo8 = l16 < 8;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const v4i P0 = pack8(0, mt, bv0), P1 = pack8(1, mt, bv1);
      v4i S, R;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        S[i] = lo8 ? P1[i] : P0[i];
        R[i] = __builtin_amdgcn_mov_dpp(S[i], 0x128 /* row_ror:8 */, 0xF, 0xF, false);
      }
      // lane r < 8 now holds row r's and row r+8's first halves; lane r+8
      // holds the second halves of rows r and r+8
      const int m = m_base + 16 * mt + l16;
      const int mA = lo8 ? m : m - 8, mB = lo8 ? m + 8 : m;
      const int nc = lo8 ? n00 : n01;
      const v4i dA = lo8 ? P0 : R, dB = lo8 ? R : P1;
      if (nc < N) {
        if (mA < M) *reinterpret_cast<v4i*>(Y + (size_t)mA * N + nc) = dA;
        if (mB < M) *reinterpret_cast<v4i*>(Y + (size_t)mB * N + nc) = dB;
      }
    }
  } else {
#pragma unroll
    for (int p2 = 0; p2 < NTW / 2; ++p2) {
      const int n0 = n_base + 32 * p2 + 8 * g;
      float bv[8];
      bias8(n0, bv);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int m = m_base + 16 * mt + l16;
        if (m >= M || n0 >= N) continue;
        *reinterpret_cast<v4i*>(Y + (size_t)m * N + n0) = pack8(p2, mt, bv);
      }
    }
  }
}

// ------------------------------------------------------------ K-B, INT4
//
// 128 (tokens) x 128 (out-features) per block of 4 waves, three blocks per
// compute unit, so each SIMD runs three waves of different blocks: one
// block's barrier or load wait is covered by the others' VALU work, and
// the tile count of a layer splits evenly over the compute units more
// often than with larger tiles.  Wave w owns tokens 64 (w & 1) .. +64 and
// out-features 64 (w >> 1) .. +64, i.e. 4 x 4 MFMA tiles of 16 x 16 (64
// fp32 accumulators per lane).  Codes travel global -> LDS by direct-to-LDS
// loads into a ring of two 16 KB step buffers, one step ahead; the scale
// records of 4 steps (token rows: one dword per step; weights: 4 rows x one
// dword per step, 64 bytes per 4-row block) are double buffered the same
// way.
//
// Each 16-byte fragment holds 16 codes of each of the step's two 64-element
// groups.  Nibbles become bytes 16 q, the int8 MFMA operand, so one MFMA per
// group gives 2^8 times the exact integer dot product I; the accumulator
// takes float(I) * (sx * sw), the fp16 scale product formed exactly in fp32,
// and the 2^8 is removed once after the K loop.
//
// After the K loop the two step buffers take the low-rank chunks (Z and
// L2'); weight rows are permuted inside tile pairs as in the MXFP4 kernel
// for 16-byte stores.

constexpr int I4_BM = 128, I4_BN = 128, I4_WAVES = 4, I4_THREADS = 64 * I4_WAVES;
constexpr int I4_STEP_BYTES = (I4_BM + I4_BN) * 64;   // codes of one step, both operands
constexpr int I4_NBUF = 2;
constexpr int I4_SC_BYTES = (I4_BM + I4_BN) * 16;     // scale records of one 4-step group
constexpr int I4_SC0 = I4_NBUF * I4_STEP_BYTES;
constexpr int I4_LDS = I4_SC0 + 2 * I4_SC_BYTES;
// after the K loop the step buffers hold a low-rank chunk: Z (128 rows x 32
// fp32) in buffer 0, L2' (128 rows x 32 bf16) in buffer 1
constexpr int I4_Z0 = 0, I4_L20 = I4_STEP_BYTES;

// product of the fp16 halves G of a and b, formed exactly in fp32 by one
// mixed-precision FMA (the fp16 inputs are widened inside it, addend 0)
template <int G>
__device__ __forceinline__ float f16_product(uint32_t a, uint32_t b) {
  float d;
  if constexpr (G == 0)
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,1,0]" : "=v"(d) : "v"(a), "v"(b));
  else
    asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,1,0] op_sel_hi:[1,1,0]" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// int8 MFMA operand of group G from a 16-byte INT4 fragment: bytes 16 q
__device__ __forceinline__ v4i i4_unpack(const v4i f, int G) {
  const uint32_t MSK = 0xF0F0F0F0u;
  const uint32_t d0 = (uint32_t)f[2 * G], d1 = (uint32_t)f[2 * G + 1];
  return (v4i){(int)((d0 << 4) & MSK), (int)(d0 & MSK), (int)((d1 << 4) & MSK), (int)(d1 & MSK)};
}

template <int NTR>
__global__ __launch_bounds__(I4_THREADS) __attribute__((amdgpu_waves_per_eu(3))) void kb_i4_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const float* __restrict__ zp,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const uint16_t* __restrict__ l2k,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int N, int K, int rpad) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[I4_LDS];
  const uint32_t lds_u32 = (uint32_t)(size_t)(SVDQ_AS3 uint8_t*)lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g = lane >> 4;
  const int tiles_m = (M + I4_BM - 1) / I4_BM, tiles_n = (N + I4_BN - 1) / I4_BN;
  int tm, tn;
  mx_tile_of(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int tile_m = tm * I4_BM, tile_n = tn * I4_BN;
  const int steps = K / 128;
  const int ks4 = (steps + 3) / 4;
  const int m_base = tile_m + 64 * wm, n_base = tile_n + 64 * wn;

  // ---- DMA plan.  Codes: 16 contiguous 1 KB units per step (units 0-7:
  // token row groups, 8-15: weight row groups); wave w moves units 4w ..
  // 4w+3, lane i 16 bytes.  Units past the last row group repeat it.
  const bool tokw = wave < 2;
  const uint8_t* cbase = tokw ? xq : wq;
  uint32_t coff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int u = 4 * (wave & 1) + j;
    const int grp16 = tokw ? min((tile_m >> 4) + u, (M + 15) / 16 - 1) : min((tile_n >> 4) + u, N / 16 - 1);
    coff[j] = (uint32_t)grp16 * (uint32_t)steps * 1024u + 16u * lane;
  }
  // Scales of 4-step group grp: waves 0-1 move the 1 KB records of token
  // rows 64 w .., waves 2-3 the two halves of the 2 KB weight-scale unit of
  // the block's 128 out-features (32 blocks of 4 rows x 4 steps).
  const uint8_t* sbase = tokw ? xs : ws;
  uint32_t soff, sstride;
  if (tokw) {
    soff = (uint32_t)min((tile_m >> 6) + wave, (M + 63) / 64 - 1) * (uint32_t)ks4 * 1024u + 16u * lane;
    sstride = 1024;
  } else {
    soff = (uint32_t)(tile_n >> 7) * (uint32_t)ks4 * 2048u + 1024u * (uint32_t)(wave & 1) + 16u * lane;
    sstride = 2048;
  }
  auto issue_codes = [&](int t) __attribute__((always_inline)) {
    const uint32_t b = lds_u32 + (uint32_t)(t % I4_NBUF) * I4_STEP_BYTES + (uint32_t)wave * 4096u;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(cbase + (size_t)t * 1024, coff[j], b + 1024u * j);
  };
  auto issue_scales = [&](int grp) __attribute__((always_inline)) {
    dma16(sbase + (size_t)grp * sstride, soff,
          lds_u32 + I4_SC0 + (uint32_t)(grp & 1) * I4_SC_BYTES + (uint32_t)wave * 1024u);
  };
  // Z (128 rows x 128 B, 16 units of 8 rows) and L2' (128 rows x 64 B, 8
  // units of 16 rows) chunk u into step buffers 0 and 1
  auto issue_lowrank = [&](int u) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int unit = 4 * wave + j, row = 8 * unit + (lane >> 3);
      const int m = min(tile_m + row, M - 1);
      dma16(reinterpret_cast<const uint8_t*>(zp),
            ((uint32_t)m * (uint32_t)rpad + 32u * u) * 4u + 16u * ((lane & 7) ^ zswz(row)),
            lds_u32 + I4_Z0 + 1024u * unit);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int unit = 2 * wave + j, row = 16 * unit + (lane >> 2);
      const int n = min(tile_n + row, N - 1);
      dma16(reinterpret_cast<const uint8_t*>(l2k),
            ((uint32_t)n * (uint32_t)rpad + 32u * u) * 2u + 16u * ((lane & 3) ^ lswz(row)),
            lds_u32 + I4_L20 + 1024u * unit);
    }
  };

  // fragment addresses inside a step buffer: token fragment q reads row
  // 64 wm + 16 q + l16 (the swizzle repeats every 32 rows), weight fragment
  // nt the permuted row 64 wn + mx_nrow(nt, l16)
  uint32_t boff[2], aoff[4];
#pragma unroll
  for (int par = 0; par < 2; ++par) boff[par] = (uint32_t)swz(64 * wm + 16 * par + l16, g) - 1024u * par;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) aoff[nt] = (uint32_t)(I4_BM * 64 + swz(64 * wn + mx_nrow(nt, l16), g));
  auto buf_of = [&](int t) __attribute__((always_inline)) -> uint32_t {
    uint32_t bo = (uint32_t)(t % I4_NBUF) * I4_STEP_BYTES;
    asm volatile("" : "+s"(bo));
    return bo;
  };
  auto read_b = [&](uint32_t bo, int q) __attribute__((always_inline)) -> v4i {
    return *reinterpret_cast<const v4i*>(lds + bo + boff[q & 1] + 1024 * q);
  };
  auto read_a = [&](uint32_t bo, int nt) __attribute__((always_inline)) -> v4i {
    return *reinterpret_cast<const v4i*>(lds + bo + aoff[nt]);
  };
  // scales of step t: token row dword (groups 2t, 2t+1) per mt; 4 weight
  // rows x dword per nt (the lane's 4 consecutive out-features)
  uint32_t sx[4];
  v4i sw[4];
  auto read_scales = [&](int t) __attribute__((always_inline)) {
    uint32_t so = (uint32_t)(I4_SC0 + ((t >> 2) & 1) * I4_SC_BYTES);
    asm volatile("" : "+s"(so));
    const uint8_t* sc = lds + so;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      sx[mt] = *reinterpret_cast<const uint32_t*>(sc + 1024 * wm + 4 * (64 * mt + 16 * (t & 3) + l16));
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int blk = 16 * wn + 8 * (nt >> 1) + 2 * g + (nt & 1);
      sw[nt] = *reinterpret_cast<const v4i*>(sc + I4_BM * 16 + blk * 64 + 16 * (t & 3));
    }
  };

  // Ring of two step buffers: the top of step t waits for step t's loads
  // and a barrier, after which step t-1's buffer (every wave is past it)
  // receives step t+1; steps 0 and 1 are issued before the loop.
  issue_scales(0);
  issue_codes(0);
  if (steps > 1) issue_codes(1);

  v4f acc[4][4];   // [weight tile][token tile]
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int t = 0; t < steps; ++t) {
    if (t == 0 && steps > 1)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t >= 1 && t + 1 < steps) issue_codes(t + 1);
    if ((t & 3) == 0 && (t >> 2) + 1 < ks4) issue_scales((t >> 2) + 1);
    read_scales(t);
    const uint32_t bc = buf_of(t);
    v4i wu[4][2], tk[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const v4i wp = read_a(bc, nt);
      wu[nt][0] = i4_unpack(wp, 0);
      wu[nt][1] = i4_unpack(wp, 1);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) tk[q] = read_b(bc, q);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int G = 0; G < 2; ++G) {
        // the group's 4 MFMAs first, then their scaling
        const v4i b8 = i4_unpack(tk[mt], G);
        v4i I[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          I[nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wu[nt][G], b8, (v4i){0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = G == 0 ? f16_product<0>(sx[mt], (uint32_t)sw[nt][i])
                                   : f16_product<1>(sx[mt], (uint32_t)sw[nt][i]);
            acc[nt][mt][i] = __builtin_fmaf((float)I[nt][i], p, acc[nt][mt][i]);
          }
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nt][mt][i] *= 1.0f / 256.0f;

  // ---- low-rank up projection and bias, then one 16-byte store per pair
  if constexpr (NTR > 0) {
    for (int u = 0; u < NTR; ++u) {
      __syncthreads();   // every wave is done with the step buffers (or chunk u-1)
      issue_lowrank(u);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      v8bf bh[4], bl[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int zrow = 64 * wm + 16 * mt + l16;
        bh[mt] = *reinterpret_cast<const v8bf*>(lds + I4_Z0 + zrow * 128 + 16 * (g ^ zswz(zrow)));
        bl[mt] = *reinterpret_cast<const v8bf*>(lds + I4_Z0 + zrow * 128 + 16 * ((4 + g) ^ zswz(zrow)));
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int lrow = 64 * wn + mx_nrow(nt, l16);
        const v8bf af = *reinterpret_cast<const v8bf*>(lds + I4_L20 + lrow * 64 + 16 * (g ^ lswz(lrow)));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh[mt], acc[nt][mt], 0, 0, 0);
          acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl[mt], acc[nt][mt], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int p2 = 0; p2 < 2; ++p2) {
    const int n0 = n_base + 32 * p2 + 8 * g;
    float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (bias != nullptr && n0 < N) {
      const v4i braw = *reinterpret_cast<const v4i*>(bias + n0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bv[2 * i] = bf16_lo((uint32_t)braw[i]);
        bv[2 * i + 1] = bf16_hi((uint32_t)braw[i]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int m = m_base + 16 * mt + l16;
      if (m >= M || n0 >= N) continue;
      v4i o;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        o[i] = (int)(bf16_rne(acc[2 * p2][mt][2 * i] + bv[2 * i]) |
                     (bf16_rne(acc[2 * p2][mt][2 * i + 1] + bv[2 * i + 1]) << 16));
        o[2 + i] = (int)(bf16_rne(acc[2 * p2 + 1][mt][2 * i] + bv[4 + 2 * i]) |
                         (bf16_rne(acc[2 * p2 + 1][mt][2 * i + 1] + bv[4 + 2 * i + 1]) << 16));
      }
      *reinterpret_cast<v4i*>(Y + (size_t)m * N + n0) = o;
    }
  }
}


// ------------------------------------------------- unfused baseline: up + add
//
// Y += Z L2' as its own pass over Y, for measuring what fusing the branch
// into the GEMM epilogue saves.  One wave per 16 tokens x 64 out-features;
// bf16 MFMA on the Z hi/lo halves and L2'^T rows, then a read-modify-write
// of the bf16 output.
template <int NTR>
__global__ __launch_bounds__(256) void kup_kernel(const uint16_t* __restrict__ zp, const uint16_t* __restrict__ l2k,
                                                  uint16_t* __restrict__ Y, int M, int N, int rpad) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int tiles_n = (N + 63) / 64, tiles = ((M + 15) / 16) * tiles_n;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= tiles) return;   // whole wave; no barriers in this kernel
  const int m0 = (tile / tiles_n) * 16, n0 = (tile % tiles_n) * 64;
  const int m = min(m0 + l16, M - 1);
  v4f acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NTR; ++u) {
    const uint16_t* zr = zp + (size_t)m * 2 * rpad + 64 * u + 8 * g;
    const v8bf bh = *reinterpret_cast<const v8bf*>(zr);
    const v8bf bl = *reinterpret_cast<const v8bf*>(zr + 32);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = min(n0 + 16 * nt + l16, N - 1);
      const v8bf af = *reinterpret_cast<const v8bf*>(l2k + (size_t)n * rpad + 32 * u + 8 * g);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl, acc[nt], 0, 0, 0);
    }
  }
  // lane holds out-features n0 + 16 nt + 4 g + 0..3 of token m0 + l16
  if (m0 + l16 >= M) return;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int nn = n0 + 16 * nt + 4 * g;
    if (nn >= N) continue;
    uint2* yp = reinterpret_cast<uint2*>(Y + (size_t)(m0 + l16) * N + nn);
    const uint2 y = *yp;
    const uint32_t lo = bf16_rne(bf16_lo(y.x) + acc[nt][0]) | (bf16_rne(bf16_hi(y.x) + acc[nt][1]) << 16);
    const uint32_t hi = bf16_rne(bf16_lo(y.y) + acc[nt][2]) | (bf16_rne(bf16_hi(y.y) + acc[nt][3]) << 16);
    *yp = make_uint2(lo, hi);
  }
}

// ------------------------------------------------------------ dispatch

// compute units of the current device, cached per device (write-once)
static std::atomic<int> g_dev_cus[64];

static int device_cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  v = g_dev_cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    g_dev_cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int FMT, int NT, bool SL, bool ZONLY, bool RING>
static void launch_ka_one(dim3 grid, dim3 block, size_t lds, hipStream_t st, const uint16_t* X, int M,
                          const svdq_layer& L, const v8bf* l1, uint8_t* xq, uint8_t* xs, float* z, int rp) {
  hipLaunchKernelGGL((ka_kernel<FMT, NT, SL, ZONLY, RING>), grid, block, lds, st, X, M, L.K, L.smooth_inv, l1, xq,
                     xs, z, rp);
}

template <int FMT, bool ZONLY = false>
static hipError_t launch_ka(const svdq_layer& L, const uint16_t* X, int M, uint8_t* ws, const svdq_ws_layout& W,
                            hipStream_t st) {
  const int rp = rank_pad(L.rank);
  dim3 grid((M + 15) / 16), block(64 * KA_WAVES);
  uint8_t* xq = ws + W.xq_off;
  uint8_t* xs = ws + W.xs_off;
  float* z = reinterpret_cast<float*>(ws + W.z_off);
  const v8bf* l1 = reinterpret_cast<const v8bf*>(L.l1k);
  // With at most one block per compute unit the register ring of down-factor
  // fragments hides their L2 latency; with more blocks than units the
  // ring-free kernel (about 110 VGPRs) runs two blocks per unit, which
  // hides it better.
  const bool ring = (int)grid.x <= device_cus();
#define SVDQ_KA(NTV)                                                                                      \
  do {                                                                                                    \
    if (L.K <= KA_SL_MAX_K) {                                                                             \
      const size_t lds = (size_t)L.K * 4;                                                                 \
      if constexpr (NTV > 0 && NTV <= 4) {                                                                \
        if (!ring) {                                                                                      \
          launch_ka_one<FMT, NTV, true, ZONLY, false>(grid, block, lds, st, X, M, L, l1, xq, xs, z, rp);  \
          break;                                                                                          \
        }                                                                                                 \
      }                                                                                                   \
      launch_ka_one<FMT, NTV, true, ZONLY, true>(grid, block, lds, st, X, M, L, l1, xq, xs, z, rp);       \
    } else {                                                                                              \
      if constexpr (NTV > 0 && NTV <= 2) {                                                                \
        if (!ring) {                                                                                      \
          launch_ka_one<FMT, NTV, false, ZONLY, false>(grid, block, 0, st, X, M, L, l1, xq, xs, z, rp);   \
          break;                                                                                          \
        }                                                                                                 \
      }                                                                                                   \
      launch_ka_one<FMT, NTV, false, ZONLY, true>(grid, block, 0, st, X, M, L, l1, xq, xs, z, rp);        \
    }                                                                                                     \
  } while (0)
  // one 16-column MFMA tile of the down factor per 16 of the rank
  switch (L.rank / 16) {
    case 0: SVDQ_KA(0); break;
    case 1: SVDQ_KA(1); break;
    case 2: SVDQ_KA(2); break;
    case 3: SVDQ_KA(3); break;
    case 4: SVDQ_KA(4); break;
    case 5: SVDQ_KA(5); break;
    case 6: SVDQ_KA(6); break;
    case 7: SVDQ_KA(7); break;
    case 8: SVDQ_KA(8); break;
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_KA
  return hipGetLastError();
}

template <int NTR, bool W8 = false>
static void launch_kb_mx(const svdq_layer& L, const uint8_t* ws, const svdq_ws_layout& W, int M, uint16_t* Y,
                         hipStream_t st) {
  const int rp = rank_pad(L.rank);
  const int tiles = ((M + MX_BM - 1) / MX_BM) * ((L.N + MX_BN - 1) / MX_BN);
  // the K loop runs in pairs of 64-byte steps; an odd step count takes the
  // variant with one trailing step (8-bit codes always have an even count)
  constexpr int WV = SVDQ_MX_WAVES;
  if constexpr (W8)
    hipLaunchKernelGGL((kb_mx_kernel<NTR, false, WV, true>), dim3(tiles), dim3(WV * 64), 0, st, ws + W.xq_off,
                       ws + W.xs_off, reinterpret_cast<const float*>(ws + W.z_off), L.wq, L.ws, L.l2k,
                       L.bias, Y, M, L.N, L.K, rp);
  else if ((L.K / 128) % 2 == 0)
    hipLaunchKernelGGL((kb_mx_kernel<NTR, false, WV>), dim3(tiles), dim3(WV * 64), 0, st, ws + W.xq_off,
                       ws + W.xs_off, reinterpret_cast<const float*>(ws + W.z_off), L.wq, L.ws, L.l2k,
                       L.bias, Y, M, L.N, L.K, rp);
  else
    hipLaunchKernelGGL((kb_mx_kernel<NTR, true, WV>), dim3(tiles), dim3(WV * 64), 0, st, ws + W.xq_off,
                       ws + W.xs_off, reinterpret_cast<const float*>(ws + W.z_off), L.wq, L.ws, L.l2k,
                       L.bias, Y, M, L.N, L.K, rp);
}

template <int FMT>
static hipError_t launch_kb(const svdq_layer& L, const uint8_t* ws, const svdq_ws_layout& W, int M, uint16_t* Y,
                            hipStream_t st) {
  const int rp = rank_pad(L.rank);
  if constexpr (FMT == SVDQ_MXFP4_G32 || FMT == SVDQ_W8A8) {
    constexpr bool W8 = FMT == SVDQ_W8A8;
    switch (rp / 32) {
      case 0: launch_kb_mx<0, W8>(L, ws, W, M, Y, st); break;
      case 1: launch_kb_mx<1, W8>(L, ws, W, M, Y, st); break;
      case 2: launch_kb_mx<2, W8>(L, ws, W, M, Y, st); break;
      case 3: launch_kb_mx<3, W8>(L, ws, W, M, Y, st); break;
      case 4: launch_kb_mx<4, W8>(L, ws, W, M, Y, st); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int tiles = ((M + I4_BM - 1) / I4_BM) * ((L.N + I4_BN - 1) / I4_BN);
  const uint8_t* xq = ws + W.xq_off;
  const uint8_t* xs = ws + W.xs_off;
  const float* zp = reinterpret_cast<const float*>(ws + W.z_off);
#define SVDQ_KB_I4(R)                                                                                          \
  hipLaunchKernelGGL((kb_i4_kernel<R>), dim3(tiles), dim3(I4_THREADS), 0, st, xq, xs, zp, L.wq, L.ws, L.l2k, \
                     L.bias, Y, M, L.N, L.K, rp)
  switch (rp / 32) {
    case 0: SVDQ_KB_I4(0); break;
    case 1: SVDQ_KB_I4(1); break;
    case 2: SVDQ_KB_I4(2); break;
    case 3: SVDQ_KB_I4(3); break;
    case 4: SVDQ_KB_I4(4); break;
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_KB_I4
  return hipGetLastError();
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static svdq_status check_layer(const svdq_layer* L, int32_t M) {
  if (!L) return SVDQ_ERR_ARG;
  if (!valid_fmt(L->fmt)) return SVDQ_ERR_UNSUPPORTED;
  if (!valid_kn(L->K, L->N) || !valid_rank(L->rank) || M < 1 || M > (1 << 20)) return SVDQ_ERR_SHAPE;
  // code buffers must stay below 2 GiB (32-bit lane offsets in the kernels)
  if ((int64_t)M * L->K > (int64_t)1 << 32 || (int64_t)L->N * L->K > (int64_t)1 << 32) return SVDQ_ERR_SHAPE;
  if (!L->smooth_inv || !L->wq || !L->ws) return SVDQ_ERR_ARG;
  if (L->rank > 0 && (!L->l1k || !L->l2k)) return SVDQ_ERR_ARG;
  if (!aligned16(L->smooth_inv) || !aligned16(L->wq) || !aligned16(L->ws) ||
      (L->rank > 0 && (!aligned16(L->l1k) || !aligned16(L->l2k))) || (L->bias && !aligned16(L->bias)))
    return SVDQ_ERR_ALIGN;
  return SVDQ_OK;
}

// gfx950 check, cached per device (write-once flags)
static std::atomic<int> g_dev_ok[64];

static svdq_status device_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SVDQ_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return svdq_device_check(dev);
  int v = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    svdq_status s = svdq_device_check(dev);
    if (s == SVDQ_ERR_DEVICE) return s;
    v = s == SVDQ_OK ? 1 : 2;
    g_dev_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED;
}

}  // namespace svdq

using namespace svdq;

extern "C" {

svdq_status svdq_device_check(int32_t device) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return SVDQ_ERR_DEVICE;
  if (device < 0 || device >= n) return SVDQ_ERR_ARG;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, device) != hipSuccess) return SVDQ_ERR_DEVICE;
  return std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED;
}

svdq_status svdq_quantize_lora_down(const svdq_layer* layer, const uint16_t* X, int32_t M, void* ws,
                                    size_t ws_bytes, void* stream) {
  svdq_status s = check_layer(layer, M);
  if (s != SVDQ_OK) return s;
  if (!X || !ws) return SVDQ_ERR_ARG;
  if (!aligned16(X) || !aligned16(ws)) return SVDQ_ERR_ALIGN;
  svdq_ws_layout W;
  if ((s = svdq_workspace_layout(M, layer->K, layer->rank, layer->fmt, &W)) != SVDQ_OK) return s;
  if (ws_bytes < W.total) return SVDQ_ERR_WORKSPACE;
  if ((s = device_ok()) != SVDQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = layer->fmt == SVDQ_MXFP4_G32
                     ? launch_ka<SVDQ_MXFP4_G32>(*layer, X, M, static_cast<uint8_t*>(ws), W, st)
                 : layer->fmt == SVDQ_W8A8 ? launch_ka<SVDQ_W8A8>(*layer, X, M, static_cast<uint8_t*>(ws), W, st)
                                           : launch_ka<SVDQ_INT4_G64>(*layer, X, M, static_cast<uint8_t*>(ws), W, st);
  return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_DEVICE;
}

svdq_status svdq_gemm_lora_up(const svdq_layer* layer, const void* ws, size_t ws_bytes, int32_t M, uint16_t* Y,
                              void* stream) {
  svdq_status s = check_layer(layer, M);
  if (s != SVDQ_OK) return s;
  if (!Y || !ws) return SVDQ_ERR_ARG;
  if (!aligned16(Y) || !aligned16(ws)) return SVDQ_ERR_ALIGN;
  svdq_ws_layout W;
  if ((s = svdq_workspace_layout(M, layer->K, layer->rank, layer->fmt, &W)) != SVDQ_OK) return s;
  if (ws_bytes < W.total) return SVDQ_ERR_WORKSPACE;
  if ((s = device_ok()) != SVDQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = layer->fmt == SVDQ_MXFP4_G32
                     ? launch_kb<SVDQ_MXFP4_G32>(*layer, static_cast<const uint8_t*>(ws), W, M, Y, st)
                 : layer->fmt == SVDQ_W8A8 ? launch_kb<SVDQ_W8A8>(*layer, static_cast<const uint8_t*>(ws), W, M, Y, st)
                                           : launch_kb<SVDQ_INT4_G64>(*layer, static_cast<const uint8_t*>(ws), W, M, Y, st);
  return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_DEVICE;
}

svdq_status svdq_linear_forward(const svdq_layer* layer, const uint16_t* X, int32_t M, uint16_t* Y, void* ws,
                                size_t ws_bytes, void* stream) {
  // validate everything for both kernels before the first launch
  svdq_status s = check_layer(layer, M);
  if (s != SVDQ_OK) return s;
  if (!X || !Y || !ws) return SVDQ_ERR_ARG;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(ws)) return SVDQ_ERR_ALIGN;
  if ((s = svdq_quantize_lora_down(layer, X, M, ws, ws_bytes, stream)) != SVDQ_OK) return s;
  return svdq_gemm_lora_up(layer, ws, ws_bytes, M, Y, stream);
}

svdq_status svdq_linear_forward_unfused(const svdq_layer* layer, const uint16_t* X, int32_t M, uint16_t* Y,
                                        void* ws, size_t ws_bytes, void* stream) {
  svdq_status s = check_layer(layer, M);
  if (s != SVDQ_OK) return s;
  if (!X || !Y || !ws) return SVDQ_ERR_ARG;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(ws)) return SVDQ_ERR_ALIGN;
  svdq_ws_layout W;
  if ((s = svdq_workspace_layout(M, layer->K, layer->rank, layer->fmt, &W)) != SVDQ_OK) return s;
  if (ws_bytes < W.total) return SVDQ_ERR_WORKSPACE;
  if ((s = device_ok()) != SVDQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  svdq_layer plain = *layer;   // the same kernels with the low-rank branch left out
  plain.rank = 0;
  const int f = layer->fmt;
  auto ka = [&](const svdq_layer& L, bool zonly) {
    if (f == SVDQ_MXFP4_G32)
      return zonly ? launch_ka<SVDQ_MXFP4_G32, true>(L, X, M, w8, W, st) : launch_ka<SVDQ_MXFP4_G32>(L, X, M, w8, W, st);
    if (f == SVDQ_W8A8)
      return zonly ? launch_ka<SVDQ_W8A8, true>(L, X, M, w8, W, st) : launch_ka<SVDQ_W8A8>(L, X, M, w8, W, st);
    return zonly ? launch_ka<SVDQ_INT4_G64, true>(L, X, M, w8, W, st) : launch_ka<SVDQ_INT4_G64>(L, X, M, w8, W, st);
  };
  hipError_t e = ka(plain, false);
  if (e == hipSuccess && layer->rank > 0) e = ka(*layer, true);
  if (e == hipSuccess)
    e = f == SVDQ_MXFP4_G32 ? launch_kb<SVDQ_MXFP4_G32>(plain, w8, W, M, Y, st)
        : f == SVDQ_W8A8    ? launch_kb<SVDQ_W8A8>(plain, w8, W, M, Y, st)
                            : launch_kb<SVDQ_INT4_G64>(plain, w8, W, M, Y, st);
  if (e == hipSuccess && layer->rank > 0) {
    const int rp = rank_pad(layer->rank);
    const int tiles = ((M + 15) / 16) * ((layer->N + 63) / 64);
    const uint16_t* zp = reinterpret_cast<const uint16_t*>(w8 + W.z_off);
    switch (rp / 32) {
      case 1: hipLaunchKernelGGL(kup_kernel<1>, dim3((tiles + 3) / 4), dim3(256), 0, st, zp, layer->l2k, Y, M, layer->N, rp); break;
      case 2: hipLaunchKernelGGL(kup_kernel<2>, dim3((tiles + 3) / 4), dim3(256), 0, st, zp, layer->l2k, Y, M, layer->N, rp); break;
      case 3: hipLaunchKernelGGL(kup_kernel<3>, dim3((tiles + 3) / 4), dim3(256), 0, st, zp, layer->l2k, Y, M, layer->N, rp); break;
      case 4: hipLaunchKernelGGL(kup_kernel<4>, dim3((tiles + 3) / 4), dim3(256), 0, st, zp, layer->l2k, Y, M, layer->N, rp); break;
      default: return SVDQ_ERR_SHAPE;
    }
    e = hipGetLastError();
  }
  return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_DEVICE;
}

}  // extern "C"
