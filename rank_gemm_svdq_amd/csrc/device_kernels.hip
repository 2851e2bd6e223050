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
//   Codes (MXFP4 and W8A8, activations and weights): 1 KB units of 16 rows
//     x one step, ordered [row / 16][step]; inside a unit, 16-byte slot
//     4 (row % 16) + q holds chunk q ^ swz(row % 32) of the row-step, in
//     canonical byte order.
//   INT4 codes: FP6 E2M3 (exact for -7..7), 32 six-bit codes of a 32-element
//     slice s = 2 G + h packed in 6 dwords; dwords 0-3 of each slice in
//     1 KB units of 16 rows x one step (slot 4 (row % 16) + (s ^ i4_swz)),
//     dwords 4-5 after all of them in 1 KB units of 32 rows x one step.
//   Scale records (MXFP4, both operands): 1 KB units of 64 rows x 4 steps
//     ordered [row / 64][4-step group]; dword d of row r sits at unit dword
//     64 (r % 64 / 16) + 16 d + r % 16 and holds the E8M0 scales of
//     32-element block d of the 4 steps (byte t % 4); the weight rows are
//     permuted inside their 64-row group (wrec_row).
//   INT4 scales: 512-byte units of 128 rows x one step, [row / 128][step]:
//     per token row one dword (the fp16 pair of the step's two groups), per
//     out-feature fp16 index 128 G + row % 128.
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
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

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

// ----------------------------------------------------------------- K-A

constexpr int KA_WAVES = 8;
constexpr int KA_SL_MAX_K = 16384;   // 1/lambda is staged in LDS up to this K

// One block handles 16 rows; its NWV waves (8, or 4 when there are more
// blocks than compute units) split the K steps evenly and the
// down-projection partial sums are reduced in LDS, so Z leaves the kernel
// once.  Lane l owns row l % 16 and the 32 consecutive elements
// 32 (l / 16) .. +32 of each 128-element step.  Each wave keeps the next
// two steps' X (and, for ranks up to 64, their down-factor fragments) in
// flight in a register ring while it processes the current one; 1/lambda
// comes from LDS when K allows.  The down projection multiplies the
// smoothed x^ = x / lambda, split into bf16 hi + lo, by the bf16 factor
// L1', so it runs on bf16 MFMA with fp32 accumulation.  ZONLY drops the
// quantisation (the unfused baseline's separate down-projection pass).
template <int FMT, int NT, bool SL, bool ZONLY = false, bool RING = true, int NWV = KA_WAVES>
__global__ __launch_bounds__(64 * NWV, 2) void ka_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                          const float* __restrict__ sinv,
                                                          const v8bf* __restrict__ l1k,
                                                          uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                                          float* __restrict__ zout, int rpad) {
  constexpr int NTZ = NT > 0 ? NT : 1;
  // down-factor fragments in the ring (RING; without them the 8-wave
  // kernel fits two blocks per unit, the W8A8 setting's choice when there
  // are more blocks than compute units)
  constexpr bool WRING = RING && NT > 0 && NT <= (SL ? 4 : 2);
  constexpr int NW = WRING ? 4 * NT : 1;
  constexpr bool W8 = FMT == SVDQ_W8A8 && !ZONLY;
  __shared__ float zred[NT > 0 ? NWV * 16 * NT * 16 : 1];
  __shared__ float mred[W8 ? NWV * 16 : 1];
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
  const size_t i4_tail = code_bytes(M, steps);   // INT4: the code tails follow the main parts
  const int spw = (steps + NWV - 1) / NWV;
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
    // each wave stages 1/lambda of its own steps, 128 (t1 - t0) floats, by
    // direct-to-LDS loads issued ahead of its X loads; only the wave itself
    // reads them (no block barrier), each read after the wait for its step's
    // X, which completes after them (loads complete in issue order)
    const uint32_t sdst = (uint32_t)(size_t)(SVDQ_AS3 float*)svl + 512u * (uint32_t)t0;
    for (int u = 0; 2 * u < t1 - t0; ++u) {
      // an odd count ends with half a kilobyte: lanes 0-31 only
      if (2 * u + 1 < t1 - t0 || lane < 32)
        dma16(reinterpret_cast<const uint8_t*>(sinv), 512u * (uint32_t)t0 + 1024u * u + 16u * lane, sdst + 1024u * u);
    }
  }
  Slot ring[2];
  if (t0 < t1) load(t0, ring[0]);
  if (t0 + 1 < t1) load(t0 + 1, ring[1]);

  v4f acc[NTZ];
#pragma unroll
  for (int nt = 0; nt < NTZ; ++nt) acc[nt] = (v4f){0.f, 0.f, 0.f, 0.f};
  float rmax = 0.f;   // W8A8: running |x^| maximum of this lane's share of its row

  // x^ = fp32(x * 1/lambda) for the lane's 32 elements of step t
  auto smooth = [&](int t, const Slot& sl, float* xh) __attribute__((always_inline)) {
    int k0 = t * 128 + 32 * g;
    if constexpr (SL) {
      // a zero that depends on this step's X: the LDS reads below cannot be
      // issued before the X loads (and the older staging loads) are done
      int dep;
      asm volatile("v_and_b32 %0, 0, %1" : "=v"(dep) : "v"(sl.x[0][0]));
      k0 += dep << 5;   // keeps the 16-byte alignment of the reads visible
    }
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
    } else if constexpr (FMT == SVDQ_MXFP4_G32 || FMT == SVDQ_MXFP4_G32_OCP) {
      // smallest e with amax <= 6 * 2^e, or with the OCP rule
      // floor(log2(amax)) - 2; clamped to [-127, 127]
      constexpr bool OCP = FMT == SVDQ_MXFP4_G32_OCP;
      const uint32_t ab = __float_as_uint(amax);
      const int ex = (int)(ab >> 23);
      int e = ex == 0 ? -127 : ex - 129 + (!OCP && (ab & 0x7FFFFFu) > 0x400000u ? 1 : 0);
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
      v4i packed;
      if (e >= -126) {
        const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
        // the OCP rule saturates at 6 2^e before the convert (exact: a
        // power-of-two multiple); x^ itself stays for the down projection
        const float lim = 6.0f * scale;
        auto sat = [&](float v) __attribute__((always_inline)) { return OCP ? fminf(fmaxf(v, -lim), lim) : v; };
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t d = 0;
          d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, sat(xh[8 * w + 0]), sat(xh[8 * w + 1]), scale, 0);
          d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, sat(xh[8 * w + 2]), sat(xh[8 * w + 3]), scale, 1);
          d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, sat(xh[8 * w + 4]), sat(xh[8 * w + 5]), scale, 2);
          d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, sat(xh[8 * w + 6]), sat(xh[8 * w + 7]), scale, 3);
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
      // fp16 scale, saturated at 65504 instead of overflowing to infinity
      _Float16 s16 = (_Float16)s32;
      if (s32 >= 65520.0f) s16 = (_Float16)65504.0f;
      const float sf = (float)s16;
      // codes -7..7 as floats, then FP6 E2M3 (exact for them): the
      // convert takes two 16-value operands and interleaves them, so the
      // even elements go in the first and the odd in the second to give
      // the dense order (element j at bits 6 j) the MFMA reads
      v16f qa, qb;
      const float rcp = sf != 0.f ? 1.0f / sf : 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        qa[j] = sf != 0.f ? fminf(fmaxf(__builtin_rintf(xh[2 * j] * rcp), -7.f), 7.f) : 0.f;
        qb[j] = sf != 0.f ? fminf(fmaxf(__builtin_rintf(xh[2 * j + 1] * rcp), -7.f), 7.f) : 0.f;
      }
      const v6i d = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(qa, qb, 1.0f);
      if (live) {
        // slice g of the step: dwords 0-3 to the main part, 4-5 to the tail
        *reinterpret_cast<v4i*>(xq + i4_main_offset(row, t, g, steps)) = (v4i){d[0], d[1], d[2], d[3]};
        *reinterpret_cast<uint2*>(xq + i4_tail + i4_tail_offset(row, t, g, steps)) =
            make_uint2((uint32_t)d[4], (uint32_t)d[5]);
        if ((g & 1) == 0) {
          uint16_t sb;
          __builtin_memcpy(&sb, &s16, 2);
          *reinterpret_cast<uint16_t*>(xs + i4_xscale_offset(row, t, g >> 1, steps)) = sb;
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
    for (int idx = threadIdx.x; idx < 16 * WP; idx += 64 * NWV) {
      const int rr = idx / WP, cc = idx % WP;
      float sum = 0.f;
      if (cc < W) {
#pragma unroll
        for (int w = 0; w < NWV; ++w) sum += zred[(w * 16 + rr) * W + cc];
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
    for (int w = 0; w < NWV; ++w) am = fmaxf(am, mred[w * 16 + r]);
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

// ----------------------------------------------------- K-B, MXFP4 and W8A8
//
// 256 (tokens) x 256 (out-features) per block of 8 waves, two per SIMD; wave
// w owns tokens 128 (w & 1) .. +128 and out-features 64 (w >> 1) .. +64, i.e.
// 4 x 8 MFMA tiles of 16 x 16 (128 fp32 accumulators per lane).  The body is
// a template on the tile side: kb_mx_kernel runs 256 x 256 tiles, and
// kb_mx_tail_kernel 128 x 128 tiles (waves own 64 tokens x 32 out-features)
// for the last columns when the large tiles would leave a mostly idle last
// round.
//
// Codes travel global -> LDS by direct-to-LDS loads (no register staging)
// into a ring of four step buffers (32 KB for the large tile); scale dwords
// (one per row and 4 steps) travel the same way into a double buffer.  The
// K loop runs in pairs of steps with one barrier per pair: the first step of
// a pair loads the next pair into the two buffers the previous pair has
// left.  The weight fragments of the next step are read into the other half
// of a two-deep register set while the current MFMAs run, and token
// fragments stream through four registers three MFMA groups ahead, so no
// fragment is ever copied between registers.  One 32-bit LDS read per 4-step
// group gives each scale register the E8M0 bytes of its four steps; it is
// shifted down by 16 bits for the group's second pair, and the MFMA's op_sel
// picks the byte.  The low-rank product Z L2' is formed before the K loop
// while the first code steps are in flight (MXFP4), or after it from Z and
// L2' tiles loaded into ring buffers the last pair no longer uses (W8A8).
//
// Weight rows are permuted inside each pair of 16-row MFMA tiles (2p, 2p+1):
// MFMA row q of tile 2p + h is out-feature 32 p + 8 (q / 4) + 4 h + q % 4, so
// the 4 + 4 accumulators a lane holds for the pair are 8 consecutive
// out-features of one token: one 16-byte store.

constexpr int MX_BM = 256, MX_BN = 256;   // the main tile; the tail tile is 128 x 128
constexpr int MX_NBUF = 4;
constexpr int MX_SC_BYTES = 8 * 1024;     // scale records of one 4-step group: one 1 KB slot per wave
// LDS plan of a TB x TB tile
template <int TB>
struct MxTile {
  static constexpr int STEP = 2 * TB * 64;                          // codes of one step, both operands
  static constexpr int DUMMY = MX_NBUF * STEP + 2 * MX_SC_BYTES;   // 1 KB per wave, see below
  static constexpr int LDS = DUMMY + 8 * 1024;
  // with the low-rank product first, the dummy region also takes the first L2' chunk (TB rows x 64 B)
  static constexpr int LDS_LRF = DUMMY + (TB * 64 > 8 * 1024 ? TB * 64 : 8 * 1024);
};

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

// The block covers out-features [n0, n1) of Y in TB-wide tiles (and all
// token rows in TB-high tiles).
template <int NTR, bool ODD, bool W8, int TB>
__device__ __forceinline__ void kb_mx_body(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                           const float* __restrict__ zp, const uint8_t* __restrict__ wq,
                                           const uint8_t* __restrict__ ws, const uint16_t* __restrict__ l2k,
                                           const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M,
                                           int N, int K, int rpad, int n0, int n1) {
  static_assert(TB == 256 || TB == 128, "tile side");
  using G = MxTile<TB>;
  constexpr int WAVES = 8;
  // LRF: the low-rank product Z L2' is formed first, while the first code
  // steps are in flight (float accumulators only, so not for W8)
  constexpr bool LRF = !W8 && NTR > 0;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LRF ? G::LDS_LRF : G::LDS];
  const uint32_t lds_u32 = (uint32_t)(size_t)(SVDQ_AS3 uint8_t*)lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves own TB/2 tokens x TB/4 out-features
  constexpr int NTW = TB / 64;           // 16-row weight tiles per wave
  constexpr int TM = TB / 32;            // 16-row token tiles per wave
  constexpr int UPW = TB / 64;           // 1 KB code units per wave and step
  constexpr int RECS = TB / 64;          // 1 KB scale records per operand and 4 steps
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g = lane >> 4;
  const int tiles_m = (M + TB - 1) / TB, tiles_n = (n1 - n0 + TB - 1) / TB;
  int tm, tn;
  mx_tile_of(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int tile_m = tm * TB, tile_n = n0 + tn * TB;
  // 64-byte code steps: 128 FP4 elements, or 64 int8 elements (W8)
  const int steps = W8 ? K / 64 : K / 128;
  const int ks4 = (steps + 3) / 4;
  const int m_base = tile_m + (TB / 2) * wm, n_base = tile_n + 16 * NTW * wn;

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
    const int grp16 = min(g0 + UPW * (wave & 3) + j, gmax);
    coff[j] = (uint32_t)grp16 * (uint32_t)steps * 1024u + 16u * lane;
  }
  // Scales: 1 KB records of 64 rows x 4 steps, RECS per operand and 4-step
  // group, into slots 0-3 (token rows) and 4-7 (weight rows) of the group's
  // buffer: wave w moves record w & 3 of its operand into slot w.  With
  // fewer than 4 records (TB = 128) the other waves re-read the last one into
  // their own slot, which nothing reads, so every wave issues one load.
  const uint8_t* sbase = tokw ? xs : ws;
  const int smax = tokw ? (M + 63) / 64 - 1 : (N + 63) / 64 - 1;
  const int grp64 = min(((tokw ? tile_m : tile_n) >> 6) + min(wave & 3, RECS - 1), smax);
  const uint32_t soff = (uint32_t)grp64 * (uint32_t)ks4 * 1024u + 16u * lane;
  const uint32_t scale_lds = lds_u32 + MX_NBUF * G::STEP;
  auto issue_codes = [&](int t) __attribute__((always_inline)) {
    const uint32_t b = lds_u32 + (uint32_t)(t % MX_NBUF) * G::STEP + (uint32_t)wave * (1024u * UPW);
#pragma unroll
    for (int j = 0; j < UPW; ++j) dma16(cbase + (size_t)t * 1024, coff[j], b + 1024u * j);
  };
  auto issue_scales = [&](int grp) __attribute__((always_inline)) {
    if constexpr (W8) return;   // W8: per-row scales, applied after the K loop
    dma16(sbase + (size_t)grp * 1024, soff, scale_lds + (uint32_t)(grp & 1) * MX_SC_BYTES + (uint32_t)wave * 1024u);
  };

  // fragment addresses (without the step-buffer offset): token fragment q
  // reads row 128 wm + 16 q + l16 (two parities, 1 KB apart per q), weight
  // fragment nt reads the permuted row 16 NTW wn + mx_nrow(nt, l16)
  uint32_t boff[2], aoff[NTW];
#pragma unroll
  for (int par = 0; par < 2; ++par) boff[par] = (uint32_t)swz((TB / 2) * wm + 16 * par + l16, g) - 1024u * par;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) aoff[nt] = (uint32_t)(TB * 64 + swz(16 * NTW * wn + mx_nrow(nt, l16), g));
  // bo: byte offset of a step buffer, kept opaque to the optimiser so that
  // it does not hoist one address register per (buffer, fragment) pair out
  // of the unrolled loop
  auto buf_of = [&](int t) __attribute__((always_inline)) -> uint32_t {
    uint32_t bo = (uint32_t)(t % MX_NBUF) * G::STEP;
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
  uint32_t asc[NTW], bsc[TM];
  auto read_scales = [&](int tp) __attribute__((always_inline)) {
    if constexpr (W8) return;
    if ((tp & 3) != 0) {
#pragma unroll
      for (int q = 0; q < TM; ++q) bsc[q] >>= 16;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) asc[nt] >>= 16;
      return;
    }
    uint32_t so = (uint32_t)(MX_NBUF * G::STEP + ((tp >> 2) & 1) * MX_SC_BYTES);
    asm volatile("" : "+s"(so));
    const uint8_t* sc = lds + so;
    // 1 KB records of 64 rows: token fragment q is rows 16 (q % 4) .. of
    // the record in slot (TB / 128) wm + q / 4; the weight records (slots
    // 4 ..) hold the fragments in order, 16 rows per tile, so the wave's
    // tile nt is 16-row block (16 NTW wn + 16 nt) % 64 / 16 of slot
    // 4 + (16 NTW wn + 16 nt) / 64; dword g of 16 rows = 256 contiguous bytes
#pragma unroll
    for (int q = 0; q < TM; ++q)
      bsc[q] = *reinterpret_cast<const uint32_t*>(sc + 1024 * ((TB / 128) * wm + (q >> 2)) +
                                                  4 * (64 * (q & 3) + 16 * g + l16));
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int wr = 16 * NTW * wn + 16 * nt;
      asc[nt] = *reinterpret_cast<const uint32_t*>(sc + 1024 * (4 + wr / 64) + 4 * (64 * ((wr & 63) >> 4) + 16 * g + l16));
    }
  };
  // The lane index is made opaque in these two so that their address
  // arithmetic is redone where they are called instead of being hoisted out
  // of the main loop into live registers.
  auto issue_z = [&](int u, uint32_t zdst) __attribute__((always_inline)) {
    // Z: TB/8 units of 8 rows x 128 B; wave w moves TB/64 of them
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j < TB / 64; ++j) {
      const int unit = (TB / 64) * wave + j, row = 8 * unit + (ln >> 3);
      const int m = min(tile_m + row, M - 1);
      dma16(reinterpret_cast<const uint8_t*>(zp),
            ((uint32_t)m * (uint32_t)rpad + 32u * u) * 4u + 16u * ((ln & 7) ^ zswz(row)), zdst + 1024u * unit);
    }
  };
  auto issue_l2 = [&](int u, uint32_t ldst) __attribute__((always_inline)) {
    // L2'^T: TB/16 units of 16 rows x 64 B; wave w moves TB/128 of them
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j < TB / 128; ++j) {
      const int unit = (TB / 128) * wave + j, row = 16 * unit + (ln >> 2);
      const int n = min(tile_n + row, N - 1);
      dma16(reinterpret_cast<const uint8_t*>(l2k),
            ((uint32_t)n * (uint32_t)rpad + 32u * u) * 2u + 16u * ((ln & 3) ^ lswz(row)), ldst + 1024u * unit);
    }
  };
  // acc += Z L2' for one 32-column chunk of the rank, from Z (rows of the
  // wave's tokens, bf16 hi and lo) and L2'^T (rows of its out-features) in LDS
  auto lr_mfma = [&](uint32_t zoff, uint32_t loff, v4f (&ac)[NTW][TM]) __attribute__((always_inline)) {
#pragma unroll
    for (int mh = 0; mh < TM / 4; ++mh) {
      v8bf bh[4], bl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int mt = 4 * mh + k;
        const int zrow = (TB / 2) * wm + 16 * mt + l16;
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

  v4f acc[NTW][TM];   // [weight tile][token tile]
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) acc[nt][mt] = (v4f){0.f, 0.f, 0.f, 0.f};

  // Prologue.  LRF: chunk 0 of Z goes to ring buffer 3 and of L2' to the
  // dummy region (neither is written by code loads before step 0 has passed
  // its barrier), ahead of the scales and code steps 0-1; the low-rank MFMAs
  // run as soon as those two have landed, while the code steps are still in
  // flight.
  constexpr uint32_t LR_Z = 3 * G::STEP, LR_L = G::DUMMY;
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
          if constexpr (UPW == 4)
            asm volatile("s_waitcnt vmcnt(9)" ::: "memory");    // 1 scale record + 2 x 4 code units
          else
            asm volatile("s_waitcnt vmcnt(5)" ::: "memory");    // 1 + 2 x 2
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
  const uint32_t zpre = (uint32_t)((t_last + 2) % MX_NBUF) * G::STEP;
  const uint32_t lpre = (uint32_t)((t_last + 3) % MX_NBUF) * G::STEP;
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
    const uint32_t cdst = more ? lds_u32 + (uint32_t)((t + 2) % MX_NBUF) * G::STEP + (uint32_t)wave * (1024u * UPW)
                               : lds_u32 + G::DUMMY + (uint32_t)wave * 1024u;
    const uint32_t cinc = more ? 1024u : 0u;
    const uint8_t* csrc2 = cbase + (size_t)(more2 ? t + 3 : steps - 1) * 1024;
    const uint32_t cdst2 = more2 ? lds_u32 + (uint32_t)((t + 3) % MX_NBUF) * G::STEP + (uint32_t)wave * (1024u * UPW)
                                 : lds_u32 + G::DUMMY + (uint32_t)wave * 1024u;
    const uint32_t cinc2 = more2 ? 1024u : 0u;
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) {
      if constexpr (!LAST) {
        // the first half of the MFMA groups loads step t+2, the second half
        // step t+3, one unit per group
        constexpr int HALF = TM / 2;
        static_assert(UPW == HALF, "one code unit per MFMA group");
        if (mt < HALF)
          dma16(csrc, coff[mt], cdst + cinc * mt);
        else
          dma16(csrc2, coff[mt - HALF], cdst2 + cinc2 * (mt - HALF));
        if (mt < NTW) wf[J ^ 1][mt] = read_a(bn, mt);
        tk[(mt + 3) & 3] = mt + 3 < TM ? read_b(bc, mt + 3) : read_b(bn, mt + 3 - TM);
      } else {
        if (mt + 3 < TM) tk[(mt + 3) & 3] = read_b(bc, mt + 3);
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
    float sxv[TM];
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) sxv[mt] = sxp[min(m_base + 16 * mt + l16, M - 1)];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sw = swp[min(n_base + mx_nrow(nt, 4 * g + i), N - 1)];
#pragma unroll
        for (int mt = 0; mt < TM; ++mt)
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
        loff = G::STEP;
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
    for (int mt = 0; mt < TM; ++mt) {
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
      const int nc0 = n_base + 32 * p2 + 8 * g;
      float bv[8];
      bias8(nc0, bv);
#pragma unroll
      for (int mt = 0; mt < TM; ++mt) {
        const int m = m_base + 16 * mt + l16;
        if (m >= M || nc0 >= N) continue;
        *reinterpret_cast<v4i*>(Y + (size_t)m * N + nc0) = pack8(p2, mt, bv);
      }
    }
  }
}

// 256 x 256 tiles over out-features [n0, n1)
template <int NTR, bool ODD, int WAVES, bool W8 = false>
__global__ __launch_bounds__(WAVES * 64, 1) void kb_mx_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const float* __restrict__ zp,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const uint16_t* __restrict__ l2k,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int N, int K, int rpad, int n0, int n1) {
  static_assert(WAVES == 8, "8 waves, two per SIMD");
  kb_mx_body<NTR, ODD, W8, 256>(xq, xs, zp, wq, ws, l2k, bias, Y, M, N, K, rpad, n0, n1);
}

// 128 x 128 tiles over out-features [n0, n1): the columns left over when
// whole rounds of 256 x 256 tiles would leave most compute units idle in a
// last, partial round
template <int NTR, bool ODD, bool W8 = false>
__global__ __launch_bounds__(512, 1) void kb_mx_tail_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const float* __restrict__ zp,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const uint16_t* __restrict__ l2k,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int N, int K, int rpad, int n0, int n1) {
  kb_mx_body<NTR, ODD, W8, 128>(xq, xs, zp, wq, ws, l2k, bias, Y, M, N, K, rpad, n0, n1);
}

// ------------------------------------------------------------ K-B, INT4
//
// 128 (tokens) x 128 (out-features) per block of 4 waves, three blocks per
// compute unit, so each SIMD runs three waves of different blocks: one
// block's barrier or load wait is covered by the others' VALU work.  Wave w
// owns tokens 64 (w & 1) .. +64 and out-features 64 (w >> 1) .. +64, i.e.
// 2 x 2 MFMA tiles of 32 x 32 (64 fp32 accumulators per lane).
//
// The codes are FP6 E2M3 values (INT4 -7..7 exactly), the operands of the
// scaled 32x32x64 MFMA (unit E8M0 scales), whose K extent is one 64-element
// group: one MFMA gives the group's exact integer dot product I as fp32.  A
// second MFMA (32x32x8 f16 with one non-zero K slot) gives the outer
// product P = sw x sx of the group's fp16 scales, exact in fp32 and in the
// same register layout, and the accumulator takes fma(I, P, acc): one VALU
// operation per output and group.  (The per-group fp16 scales are not
// powers of two, so they cannot ride in the MFMA's block scales.)
//
// Each step (128 elements = 2 groups) travels global -> LDS by direct-to-LDS
// loads into a ring of two 25.5 KB step buffers, one step ahead: the code
// main parts (16 + 16 units of 1 KB), the code tails (4 + 4 units) and the
// step's scales (512 B of token rows, 512 B of weight rows), followed by a
// 512-byte zero pad that no load writes.
//
// Weight rows are read in a permuted order inside each 32-row tile: MFMA row
// q holds out-feature i4_nrow(q), so the 16 accumulators a lane holds for a
// tile are 16 consecutive out-features of one token (two 16-byte stores).

constexpr int I4_BM = 128, I4_BN = 128, I4_WAVES = 4, I4_THREADS = 64 * I4_WAVES;
// step buffer: token main | weight main | token tails | weight tails | token scales | weight scales
constexpr int I4_BMAIN = 0, I4_AMAIN = 8192, I4_BTAIL = 16384, I4_ATAIL = 20480, I4_BSC = 24576, I4_ASC = 25088;
// then 512 zero bytes that no load writes: lanes 32-63 read their (zero)
// scale-product operands there, so the loop selects nothing per lane
constexpr int I4_ZPAD = 25600, I4_STEP_BYTES = 26112;
constexpr int I4_LDS = 2 * I4_STEP_BYTES;
// after the K loop: Z (128 rows x 32 hi + 32 lo bf16) in buffer 0, L2' (128 rows x 32 bf16) in buffer 1
constexpr int I4_Z0 = 0, I4_L20 = I4_STEP_BYTES;

// out-feature (within a 32-row tile) of MFMA row q: the 32x32 result puts
// rows 8 a + 4 h + b (a, b < 4) in lane half h, register 4 a + b, so out-feature
// 16 h + 4 a + b makes register i of a lane out-feature 16 h + i
__device__ __forceinline__ int i4_nrow(int q) { return 16 * ((q >> 2) & 1) + 4 * (q >> 3) + (q & 3); }

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
  const int l32 = lane & 31, h = lane >> 5;
  const int tiles_m = (M + I4_BM - 1) / I4_BM, tiles_n = (N + I4_BN - 1) / I4_BN;
  int tm, tn;
  mx_tile_of(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int tile_m = tm * I4_BM, tile_n = tn * I4_BN;
  const int steps = K / 128;
  const int m_base = tile_m + 64 * wm, n_base = tile_n + 64 * wn;

  // ---- DMA plan.  24 code units of 1 KB per step (0-7 token main row
  // groups of 16, 8-15 weight main, 16-19 token tails of 32 rows, 20-23
  // weight tails); wave w moves units 6 w .. 6 w + 5, lane i 16 bytes.  Row
  // groups past the last repeat it (their outputs are never stored).
  // Consecutive steps of a row group are 1 KB apart in every part.
  const uint8_t* xtail = xq + code_bytes(M, steps);
  const uint8_t* wtail = wq + code_bytes(N, steps);
  const uint8_t* ubase[6];
  uint32_t udst[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int u = 6 * wave + j;
    const uint8_t* b;
    uint32_t dst;
    if (u < 8) {
      b = xq + (size_t)min((tile_m >> 4) + u, (M + 15) / 16 - 1) * steps * 1024;
      dst = I4_BMAIN + 1024u * u;
    } else if (u < 16) {
      b = wq + (size_t)min((tile_n >> 4) + u - 8, N / 16 - 1) * steps * 1024;
      dst = I4_AMAIN + 1024u * (u - 8);
    } else if (u < 20) {
      b = xtail + (size_t)min((tile_m >> 5) + u - 16, (M + 31) / 32 - 1) * steps * 1024;
      dst = I4_BTAIL + 1024u * (u - 16);
    } else {
      b = wtail + (size_t)min((tile_n >> 5) + u - 20, (N + 31) / 32 - 1) * steps * 1024;
      dst = I4_ATAIL + 1024u * (u - 20);
    }
    ubase[j] = b;
    udst[j] = dst;
  }
  // the step's scales: 512 B of token rows (lanes 0-31) and 512 B of weight
  // rows (lanes 32-63), both moved by wave 0
  const uint8_t* sx_base = xs + (size_t)tm * steps * 512;
  const uint8_t* sw_base = ws + (size_t)tn * steps * 512;
  auto issue_step = [&](int t) __attribute__((always_inline)) {
    const uint32_t b = lds_u32 + (uint32_t)(t & 1) * I4_STEP_BYTES;
#pragma unroll
    for (int j = 0; j < 6; ++j) dma16(ubase[j] + (size_t)t * 1024, 16u * lane, b + udst[j]);
    if (wave == 0) {
      if (lane < 32)
        dma16(sx_base + (size_t)t * 512, 16u * lane, b + I4_BSC);
      else
        dma16(sw_base + (size_t)t * 512, 16u * (lane - 32), b + I4_BSC);
    }
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

  // the zero pads of both step buffers (visible after the loop's first barrier)
  if (tid < 2 * 128) *reinterpret_cast<uint32_t*>(lds + (tid >> 7) * I4_STEP_BYTES + I4_ZPAD + 4 * (tid & 127)) = 0u;
  // scale offsets inside a step buffer: a token row's fp16 pair (+ 128 per
  // token tile) and a weight row's fp16 (+ 64 per weight tile, + 256 per
  // group); lanes 32-63 point at the zero pad
  const uint32_t sxo = h ? (uint32_t)I4_ZPAD : (uint32_t)(I4_BSC + 4 * (64 * wm + l32));
  const uint32_t swo = h ? (uint32_t)I4_ZPAD : (uint32_t)(I4_ASC + 2 * (64 * wn + i4_nrow(l32)));
  // fragment offsets inside a step buffer, per tile and group G: the main
  // part of slice 2 G + h of the row, and its tail
  // (the second tile's main parts sit 2048 bytes after the first's: the
  // loop forms one base per operand, group and step and reaches the second
  // tile through the LDS instruction's immediate offset)
  uint32_t amain[2][2], atail[2], bmain[2][2], btail[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ra = 64 * wn + 32 * i + i4_nrow(l32), rb = 64 * wm + 32 * i + l32;
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      amain[i][G] = I4_AMAIN + 64 * ra + 16 * ((2 * G + h) ^ i4_swz(ra));
      bmain[i][G] = I4_BMAIN + 64 * rb + 16 * ((2 * G + h) ^ i4_swz(rb));
    }
    atail[i] = I4_ATAIL + 1024 * (ra >> 5) + 256 * h + 8 * (ra & 31);
    btail[i] = I4_BTAIL + 1024 * (rb >> 5) + 256 * h + 8 * (rb & 31);
  }
  auto buf_of = [&](int t) __attribute__((always_inline)) -> uint32_t {
    uint32_t bo = (uint32_t)(t & 1) * I4_STEP_BYTES;
    asm volatile("" : "+s"(bo));
    return bo;
  };
  auto frag = [&](uint32_t bo, uint32_t mo, uint32_t to) __attribute__((always_inline)) -> v8i {
    const v4i m4 = *reinterpret_cast<const v4i*>(lds + mo);
    // an opaque address per tail read keeps the compiler from merging two
    // tails into one ds_read2 and then copying them into the operands
    uint32_t ta = bo + to;
    asm volatile("" : "+v"(ta));
    const uint2 t2 = *reinterpret_cast<const uint2*>(lds + ta);
    return (v8i){m4[0], m4[1], m4[2], m4[3], (int)t2.x, (int)t2.y, 0, 0};
  };

  issue_step(0);
  v16f acc[2][2];   // [weight tile][token tile]
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nt][mt][i] = 0.f;

  for (int t = 0; t < steps; ++t) {
    // step t has landed; every wave is past step t - 1, whose buffer now
    // receives step t + 1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < steps) issue_step(t + 1);
    const uint32_t bo = buf_of(t);
    // this step's bases of the main parts (per operand and group) and of the
    // scales; the tails keep one address per read (frag)
    uint32_t vam[2] = {bo + amain[0][0], bo + amain[0][1]}, vbm[2] = {bo + bmain[0][0], bo + bmain[0][1]};
    uint32_t vsx = bo + sxo, vsw = bo + swo;
    asm volatile("" : "+v"(vam[0]), "+v"(vam[1]), "+v"(vbm[0]), "+v"(vbm[1]), "+v"(vsx), "+v"(vsw));
    // token scales: the fp16 pair (group 0, group 1) of the lane's token per tile
    uint32_t sx[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      sx[mt] = *reinterpret_cast<const uint32_t*>(lds + vsx + 128 * mt);
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      v8i af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = frag(bo, vam[G] + 2048 * i, atail[i] + 512 * G);
        bf[i] = frag(bo, vbm[G] + 2048 * i, btail[i] + 512 * G);
      }
      // operands of the scale-product MFMA (32x32x8 f16, K slot 0 only):
      // lanes 0-31 hold the fp16 scale of their weight row (MFMA row order)
      // or token in element 0, every other element is zero (lanes 32-63
      // read the zero pad), so the product is the outer product sw x sx,
      // exact in fp32
      v4h pa[2], pb[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint32_t w = *reinterpret_cast<const uint16_t*>(lds + vsw + 256 * G + 64 * nt);
        pa[nt] = __builtin_bit_cast(v4h, (v2i){(int)w, 0});
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint32_t x = G == 0 ? (sx[mt] & 0xFFFFu) : (sx[mt] >> 16);
        pb[mt] = __builtin_bit_cast(v4h, (v2i){(int)x, 0});
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const v16f I = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[nt], bf[mt], (v16f){}, 2, 2, 0, 127, 0,
                                                                          127);
          const v16f P = __builtin_amdgcn_mfma_f32_32x32x8f16(pa[nt], pb[mt], (v16f){}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[nt][mt][i] = __builtin_fmaf(I[i], P[i], acc[nt][mt][i]);
        }
    }
  }

  // ---- low-rank up projection and bias, then two 16-byte stores per tile
  if constexpr (NTR > 0) {
    for (int u = 0; u < NTR; ++u) {
      __syncthreads();   // every wave is done with the step buffers (or chunk u-1)
      issue_lowrank(u);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      // bf16 32x32x16 MFMAs: lane l supplies row l % 32 and the 8 values
      // k = 16 j + 8 (l / 32) .. +8 of the chunk's K half j; Z as hi and lo
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = 2 * j + h;
        v8bf zh[2], zl[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int zrow = 64 * wm + 32 * mt + l32;
          zh[mt] = *reinterpret_cast<const v8bf*>(lds + I4_Z0 + zrow * 128 + 16 * (c ^ zswz(zrow)));
          zl[mt] = *reinterpret_cast<const v8bf*>(lds + I4_Z0 + zrow * 128 + 16 * ((4 + c) ^ zswz(zrow)));
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int lrow = 64 * wn + 32 * nt + i4_nrow(l32);
          const v8bf lf = *reinterpret_cast<const v8bf*>(lds + I4_L20 + lrow * 64 + 16 * (c ^ lswz(lrow)));
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf, zh[mt], acc[nt][mt], 0, 0, 0);
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf, zl[mt], acc[nt][mt], 0, 0, 0);
          }
        }
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n0 = n_base + 32 * nt + 16 * h;
    float bv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) bv[i] = 0.f;
    if (bias != nullptr && n0 < N) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const v4i braw = *reinterpret_cast<const v4i*>(bias + n0 + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bv[8 * c + 2 * i] = bf16_lo((uint32_t)braw[i]);
          bv[8 * c + 2 * i + 1] = bf16_hi((uint32_t)braw[i]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int m = m_base + 32 * mt + l32;
      if (m >= M || n0 >= N) continue;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        v4i o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = (int)(bf16_rne(acc[nt][mt][8 * c + 2 * i] + bv[8 * c + 2 * i]) |
                       (bf16_rne(acc[nt][mt][8 * c + 2 * i + 1] + bv[8 * c + 2 * i + 1]) << 16));
        *reinterpret_cast<v4i*>(Y + (size_t)m * N + n0 + 8 * c) = o;
      }
    }
  }
}


// ------------------------------------------------- unfused baseline: up + add
//
// Y += Z L2' as its own pass over Y, for measuring what fusing the branch
// into the GEMM epilogue saves.  A block of 4 waves covers 64 tokens x 256
// out-features as four 64-wide sub-tiles: wave w loads the Z fragments
// (hi and lo) of tokens 16 w .. +16 once and forms each sub-tile's products
// on bf16 MFMA against L2'^T rows; the fp32 products pass through LDS, and
// the read-modify-write of Y runs with 8 consecutive bf16 per lane, so
// every load and store instruction covers whole 128-byte lines of Y rows.
constexpr int KUP_LD = 68;    // LDS row stride (floats) of the 64 x 64 product tile
constexpr int KUP_SUB = 4;    // 64-wide sub-tiles per block

template <int NTR>
__global__ __launch_bounds__(256) void kup_kernel(const uint16_t* __restrict__ zp, const uint16_t* __restrict__ l2k,
                                                  uint16_t* __restrict__ Y, int M, int N, int rpad) {
  __shared__ float tile[64 * KUP_LD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int tiles_n = (N + 64 * KUP_SUB - 1) / (64 * KUP_SUB);
  const int m0 = (blockIdx.x / tiles_n) * 64, n0 = (blockIdx.x % tiles_n) * (64 * KUP_SUB);
  const int m = min(m0 + 16 * wave + l16, M - 1);
  // the wave's Z fragments, reused by every sub-tile
  v8bf bh[NTR], bl[NTR];
#pragma unroll
  for (int u = 0; u < NTR; ++u) {
    const uint16_t* zr = zp + (size_t)m * 2 * rpad + 64 * u + 8 * g;
    bh[u] = *reinterpret_cast<const v8bf*>(zr);
    bl[u] = *reinterpret_cast<const v8bf*>(zr + 32);
  }
  for (int sub = 0; sub < KUP_SUB; ++sub) {
    const int ns = n0 + 64 * sub;
    if (ns >= N) break;   // uniform over the block
    // 512 pieces of 8 outputs: row c / 8, columns 8 (c % 8) .. +8; the
    // thread's two pieces of Y are loaded before the products are formed,
    // so that their latency overlaps the L2' loads and MFMAs (each piece is
    // read and written by this thread only)
    v4i yin[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = (int)threadIdx.x + 256 * j, row = c >> 3, col = 8 * (c & 7);
      const int mm = m0 + row, nn = ns + col;
      yin[j] = (mm < M && nn < N) ? *reinterpret_cast<const v4i*>(Y + (size_t)mm * N + nn) : (v4i){0, 0, 0, 0};
    }
    v4f acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NTR; ++u) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int n = min(ns + 16 * nt + l16, N - 1);
        const v8bf af = *reinterpret_cast<const v8bf*>(l2k + (size_t)n * rpad + 32 * u + 8 * g);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh[u], acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl[u], acc[nt], 0, 0, 0);
      }
    }
    // lane holds out-features 16 nt + 4 g + i of token 16 wave + l16
    if (sub > 0) __syncthreads();   // the previous sub-tile's reads of the tile are done
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      *reinterpret_cast<v4f*>(&tile[(16 * wave + l16) * KUP_LD + 16 * nt + 4 * g]) = acc[nt];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = (int)threadIdx.x + 256 * j, row = c >> 3, col = 8 * (c & 7);
      const int mm = m0 + row, nn = ns + col;
      if (mm >= M || nn >= N) continue;
      v4i* yp = reinterpret_cast<v4i*>(Y + (size_t)mm * N + nn);
      const v4i y = yin[j];
      const float* a = &tile[row * KUP_LD + col];
      v4i o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = (int)(bf16_rne(bf16_lo((uint32_t)y[i]) + a[2 * i]) | (bf16_rne(bf16_hi((uint32_t)y[i]) + a[2 * i + 1]) << 16));
      *yp = o;
    }
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

template <int FMT, int NT, bool SL, bool ZONLY, bool RING, int NWV = KA_WAVES>
static void launch_ka_one(dim3 grid, size_t lds, hipStream_t st, const uint16_t* X, int M, const svdq_layer& L,
                          const v8bf* l1, uint8_t* xq, uint8_t* xs, float* z, int rp) {
  hipLaunchKernelGGL((ka_kernel<FMT, NT, SL, ZONLY, RING, NWV>), grid, dim3(64 * NWV), lds, st, X, M, L.K,
                     L.smooth_inv, l1, xq, xs, z, rp);
}

template <int FMT, bool ZONLY = false>
static hipError_t launch_ka(const svdq_layer& L, const uint16_t* X, int M, uint8_t* ws, const svdq_ws_layout& W,
                            hipStream_t st) {
  const int rp = rank_pad(L.rank);
  dim3 grid((M + 15) / 16);
  uint8_t* xq = ws + W.xq_off;
  uint8_t* xs = ws + W.xs_off;
  float* z = reinterpret_cast<float*>(ws + W.z_off);
  const v8bf* l1 = reinterpret_cast<const v8bf*>(L.l1k);
  // With at most one block per compute unit the register ring of down-factor
  // fragments hides their L2 latency.  With more blocks than units, blocks
  // of 4 waves keep the ring (two blocks per unit, two waves per SIMD, each
  // wave with twice the K steps to pipeline); blocks of 8 would either drop
  // to one block per unit or, without the ring, wait for every step's
  // fragments where they are used.  W8A8, whose second pass over X makes
  // each wave's chain longer, keeps the ring-free 8-wave blocks (two per
  // unit), measured slightly faster there.
  const bool ring = (int)grid.x <= device_cus();
  constexpr bool W8P = FMT == SVDQ_W8A8 && !ZONLY;
#define SVDQ_KA(NTV)                                                                                      \
  do {                                                                                                    \
    if (L.K <= KA_SL_MAX_K) {                                                                             \
      const size_t lds = (size_t)L.K * 4;                                                                 \
      if constexpr (NTV > 0 && NTV <= 4) {                                                                \
        if (!ring) {                                                                                      \
          if constexpr (W8P)                                                                              \
            launch_ka_one<FMT, NTV, true, ZONLY, false>(grid, lds, st, X, M, L, l1, xq, xs, z, rp);       \
          else                                                                                            \
            launch_ka_one<FMT, NTV, true, ZONLY, true, 4>(grid, lds, st, X, M, L, l1, xq, xs, z, rp);     \
          break;                                                                                          \
        }                                                                                                 \
      }                                                                                                   \
      launch_ka_one<FMT, NTV, true, ZONLY, true>(grid, lds, st, X, M, L, l1, xq, xs, z, rp);              \
    } else {                                                                                              \
      if constexpr (NTV > 0 && NTV <= 2) {                                                                \
        if (!ring) {                                                                                      \
          if constexpr (W8P)                                                                              \
            launch_ka_one<FMT, NTV, false, ZONLY, false>(grid, 0, st, X, M, L, l1, xq, xs, z, rp);        \
          else                                                                                            \
            launch_ka_one<FMT, NTV, false, ZONLY, true, 4>(grid, 0, st, X, M, L, l1, xq, xs, z, rp);      \
          break;                                                                                          \
        }                                                                                                 \
      }                                                                                                   \
      launch_ka_one<FMT, NTV, false, ZONLY, true>(grid, 0, st, X, M, L, l1, xq, xs, z, rp);               \
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

// Out-features covered by 256-wide tiles; the rest go to 128-wide tiles.
// When the 256 x 256 tiles leave a last round that fills at most a quarter
// of the compute units, whole 256-wide columns are kept for the full rounds
// and the remaining columns are cut into 128 x 128 tiles (four per 256 x 256
// tile), one round of them over all units.  A 128 x 128 tile does about half
// the work per unit time of a 256 x 256 one (eight waves with a quarter of
// the MFMAs each per barrier), so it only pays against a mostly idle round.
static int kb_mx_main_cols(int M, int N) {
  const int cus = device_cus();
  const int tm = (M + MX_BM - 1) / MX_BM, tn = (N + MX_BN - 1) / MX_BN, tiles = tm * tn;
  const int tail = tiles % cus;
  if (tiles <= cus || tail == 0 || 4 * tail > cus) return N;
  const int cols = (tiles / cus) * cus / tm;   // 256-wide columns within the full rounds
  return cols >= tn ? N : cols * MX_BN;
}

template <int NTR, bool W8 = false>
static void launch_kb_mx(const svdq_layer& L, const uint8_t* ws, const svdq_ws_layout& W, int M, uint16_t* Y,
                         hipStream_t st) {
  const int rp = rank_pad(L.rank);
  const int n_main = kb_mx_main_cols(M, L.N);
  const int tiles = ((M + MX_BM - 1) / MX_BM) * ((n_main + MX_BN - 1) / MX_BN);
  const int tail_tiles = ((M + 127) / 128) * ((L.N - n_main + 127) / 128);
  const uint8_t *xq = ws + W.xq_off, *xs = ws + W.xs_off;
  const float* zp = reinterpret_cast<const float*>(ws + W.z_off);
  // the K loop runs in pairs of 64-byte steps; an odd step count takes the
  // variant with one trailing step (8-bit codes always have an even count)
  const bool odd = (L.K / 128) % 2 != 0;
#define SVDQ_KB_MX(ODDV)                                                                                         \
  do {                                                                                                           \
    if (tiles > 0)                                                                                               \
      hipLaunchKernelGGL((kb_mx_kernel<NTR, ODDV, 8, W8>), dim3(tiles), dim3(512), 0, st, xq, xs, zp, L.wq, L.ws, \
                         L.l2k, L.bias, Y, M, L.N, L.K, rp, 0, n_main);                                          \
    if (tail_tiles > 0)                                                                                          \
      hipLaunchKernelGGL((kb_mx_tail_kernel<NTR, ODDV, W8>), dim3(tail_tiles), dim3(512), 0, st, xq, xs, zp, L.wq, \
                         L.ws, L.l2k, L.bias, Y, M, L.N, L.K, rp, n_main, L.N);                                  \
  } while (0)
  if constexpr (W8) {
    SVDQ_KB_MX(false);
  } else {
    if (odd)
      SVDQ_KB_MX(true);
    else
      SVDQ_KB_MX(false);
  }
#undef SVDQ_KB_MX
}

template <int FMT>
static hipError_t launch_kb(const svdq_layer& L, const uint8_t* ws, const svdq_ws_layout& W, int M, uint16_t* Y,
                            hipStream_t st) {
  const int rp = rank_pad(L.rank);
  if constexpr (FMT == SVDQ_MXFP4_G32 || FMT == SVDQ_MXFP4_G32_OCP || FMT == SVDQ_W8A8) {
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

// call fn with the format as a compile-time constant
template <class Fn>
static hipError_t by_format(int fmt, Fn&& fn) {
  switch (fmt) {
    case SVDQ_INT4_G64: return fn(std::integral_constant<int, SVDQ_INT4_G64>{});
    case SVDQ_MXFP4_G32: return fn(std::integral_constant<int, SVDQ_MXFP4_G32>{});
    case SVDQ_MXFP4_G32_OCP: return fn(std::integral_constant<int, SVDQ_MXFP4_G32_OCP>{});
    case SVDQ_W8A8: return fn(std::integral_constant<int, SVDQ_W8A8>{});
  }
  return hipErrorInvalidValue;
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

// Workspace of svdq_linear_forward_noalloc: one file-scope device array per
// GPU (the runtime places a copy on every device the library runs on, held
// until the process ends).  Its name is only a host-side stand-in: host code
// uses the device address hipGetSymbolAddress returns, looked up once per
// device with that device current and kept here.
static __device__ __align__(256) uint8_t scratch[SVDQ_NOALLOC_MAX_WORKSPACE];
static std::atomic<uint8_t*> g_scratch[64];

static svdq_status scratch_of_current_device(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SVDQ_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return SVDQ_ERR_UNSUPPORTED;
  uint8_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return SVDQ_ERR_DEVICE;
    p = static_cast<uint8_t*>(q);
    g_scratch[dev].store(p, std::memory_order_release);   // racing first calls store the same address
  }
  *out = p;
  return SVDQ_OK;
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
  const hipError_t e = by_format(layer->fmt, [&](auto f) {
    return launch_ka<decltype(f)::value>(*layer, X, M, static_cast<uint8_t*>(ws), W, st);
  });
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
  const hipError_t e = by_format(layer->fmt, [&](auto f) {
    return launch_kb<decltype(f)::value>(*layer, static_cast<const uint8_t*>(ws), W, M, Y, st);
  });
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

svdq_status svdq_linear_forward_noalloc(const svdq_layer* layer, const uint16_t* X, int32_t M, uint16_t* Y,
                                        void* stream) {
  svdq_status s = check_layer(layer, M);
  if (s != SVDQ_OK) return s;
  if (!X || !Y) return SVDQ_ERR_ARG;
  if (!aligned16(X) || !aligned16(Y)) return SVDQ_ERR_ALIGN;
  svdq_ws_layout W;
  if ((s = svdq_workspace_layout(M, layer->K, layer->rank, layer->fmt, &W)) != SVDQ_OK) return s;
  if (W.total > (size_t)SVDQ_NOALLOC_MAX_WORKSPACE) return SVDQ_ERR_WORKSPACE;
  if ((s = device_ok()) != SVDQ_OK) return s;
  uint8_t* ws = nullptr;
  if ((s = scratch_of_current_device(&ws)) != SVDQ_OK) return s;
  // the same kernels as svdq_linear_forward, with the scratch array as the
  // workspace (nothing in it needs clearing: K-A writes every byte K-B reads
  // for the M rows, and rows past M are never stored)
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = by_format(layer->fmt, [&](auto f) {
    constexpr int F = decltype(f)::value;
    const hipError_t ea = launch_ka<F>(*layer, X, M, ws, W, st);
    return ea == hipSuccess ? launch_kb<F>(*layer, ws, W, M, Y, st) : ea;
  });
  return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_DEVICE;
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
  hipError_t e = by_format(layer->fmt, [&](auto f) {
    constexpr int F = decltype(f)::value;
    hipError_t r = launch_ka<F>(plain, X, M, w8, W, st);                    // quantize only
    if (r == hipSuccess && layer->rank > 0) r = launch_ka<F, true>(*layer, X, M, w8, W, st);   // down projection
    if (r == hipSuccess) r = launch_kb<F>(plain, w8, W, M, Y, st);           // GEMM + bias, Y stored
    return r;
  });
  if (e == hipSuccess && layer->rank > 0) {
    const int rp = rank_pad(layer->rank);
    const int tiles = ((M + 63) / 64) * ((layer->N + 64 * KUP_SUB - 1) / (64 * KUP_SUB));
    const uint16_t* zp = reinterpret_cast<const uint16_t*>(w8 + W.z_off);
    switch (rp / 32) {
      case 1: hipLaunchKernelGGL(kup_kernel<1>, dim3(tiles), dim3(256), 0, st, zp, layer->l2k, Y, M, layer->N, rp); break;
      case 2: hipLaunchKernelGGL(kup_kernel<2>, dim3(tiles), dim3(256), 0, st, zp, layer->l2k, Y, M, layer->N, rp); break;
      case 3: hipLaunchKernelGGL(kup_kernel<3>, dim3(tiles), dim3(256), 0, st, zp, layer->l2k, Y, M, layer->N, rp); break;
      case 4: hipLaunchKernelGGL(kup_kernel<4>, dim3(tiles), dim3(256), 0, st, zp, layer->l2k, Y, M, layer->N, rp); break;
      default: return SVDQ_ERR_SHAPE;
    }
    e = hipGetLastError();
  }
  return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_DEVICE;
}

}  // extern "C"
