// Sustained matrix-unit rate of the device: a diagnostic for pricing the
// GEMM kernels against what the chip delivers, beside the datasheet peak.
// Not part of the layer.
//
// Every block (512 threads, two waves per SIMD) issues MFMAs back to back
// with independent accumulators, on operands that change every MFMA (four
// register sets of bytes from a fixed integer hash, or all zero) and with no
// memory traffic inside the timed loop.  The matrix units' power draw
// depends on how much their operands toggle, and the shader clock is set by
// power management, so random and zero operands bracket what real data can
// reach.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "host_internal.h"

namespace svdq {

typedef int p4i __attribute__((ext_vector_type(4)));
typedef int p8i __attribute__((ext_vector_type(8)));
typedef float p4f __attribute__((ext_vector_type(4)));
typedef int p16i __attribute__((ext_vector_type(16)));

static __device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// KIND 0: scaled 16x16x128 FP4 (E2M1, unit E8M0 scales), 32 per wave and
// iteration; KIND 1: 32x32x32 int8, 16 per wave and iteration.  Both are
// 65536 operations per MFMA.
template <int KIND>
__global__ __launch_bounds__(512) void mfma_rate_kernel(int zero, int iters, float* __restrict__ sink,
                                                        uint64_t* __restrict__ marks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  p8i A[4], B[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t base = (uint32_t)blockIdx.x * 4096u + (uint32_t)threadIdx.x * 8u + (uint32_t)i;
      A[s][i] = zero ? 0 : (int)mix32(base * 2u + 1u + 977u * (uint32_t)s);
      B[s][i] = zero ? 0 : (int)mix32(base * 2u + 2u + 1931u * (uint32_t)s);
    }
  p4f acc[8];
  p16i iacc[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = (p4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) iacc[i] = (p16i){};
  __syncthreads();
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (KIND == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[(s + i) & 3], B[(s + 2 * i) & 3], acc[i], 4, 4,
                                                                     0, 127, 0, 127);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const p8i a = A[(s + i) & 3], b = B[(s + 2 * i) & 3];
          iacc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8((p4i){a[0], a[1], a[2], a[3]}, (p4i){b[0], b[1], b[2], b[3]},
                                                          iacc[i], 0, 0, 0);
        }
      }
    }
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) v += acc[i][0];
#pragma unroll
  for (int i = 0; i < 4; ++i) v += (float)iacc[i][0];
  sink[(size_t)blockIdx.x * 512 + threadIdx.x] = v;
  if (marks != nullptr && lane == 0) {
    marks[((size_t)blockIdx.x * 8 + wave) * 2 + 0] = c1 - c0;
    marks[((size_t)blockIdx.x * 8 + wave) * 2 + 1] = r1 - r0;
  }
}

}  // namespace svdq

extern "C" svdq_status svdq_mfma_rate_probe(int32_t kind, int32_t zero_operands, int32_t blocks, int32_t iters,
                                            float* sink, uint64_t* marks, void* stream) {
  if (kind < 0 || kind > 1 || blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 20) || sink == nullptr)
    return SVDQ_ERR_ARG;
  if (((uintptr_t)sink & 3u) != 0 || ((uintptr_t)marks & 7u) != 0) return SVDQ_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SVDQ_ERR_DEVICE;
  const svdq_status s = svdq_device_check(dev);
  if (s != SVDQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int z = zero_operands != 0;
  if (kind == 0)
    hipLaunchKernelGGL(svdq::mfma_rate_kernel<0>, dim3(blocks), dim3(512), 0, st, z, iters, sink, marks);
  else
    hipLaunchKernelGGL(svdq::mfma_rate_kernel<1>, dim3(blocks), dim3(512), 0, st, z, iters, sink, marks);
  return hipGetLastError() == hipSuccess ? SVDQ_OK : SVDQ_ERR_DEVICE;
}
