// Smooth-factor grid search of one layer (AutoRound doc, "Smooth search"):
// every candidate (alpha, beta) is prepared on the host, copied into one
// set of device layer buffers and scored by running the fused forward on
// the calibration rows against the floating-point output X W.  With
// residual iteration, every iteration of a candidate is scored that way and
// the best one kept (AutoRound doc, "Residual iteration": calibration
// output error when smooth is on).
//
// Device work per search: the per-channel absolute maximum of the
// calibration rows (the activation statistic of lambda), the fp32 reference
// X W once, and per candidate the forward plus one squared-difference
// reduction.  Reductions write per-block fp64 partial sums that the host
// adds in a fixed order, so the scores are deterministic.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "host_internal.h"

namespace svdq {

constexpr int SR_BLOCKS = 1024;   // partial sums per reduction
constexpr int AMAX_ROWS = 64;     // calibration rows per block of the absmax pass

// Pass 1 of the channel absmax: block (cb, rb) covers channels 256 cb ..
// +256 and rows 64 rb .. +64; the maximum goes to part[rb][k] as fp32 bits
// (non-negative floats order like their bits).  A NaN or Inf input is
// recorded as +Inf.
__global__ __launch_bounds__(256) void amax_part_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                        uint32_t* __restrict__ part) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const int r0 = blockIdx.y * AMAX_ROWS, r1 = min(M, r0 + AMAX_ROWS);
  uint32_t m = 0;
  for (int r = r0; r < r1; ++r) {
    const uint32_t h = x[(size_t)r * K + k];
    const uint32_t a = (h & 0x7F80u) == 0x7F80u ? 0x7F800000u : (h & 0x7FFFu) << 16;
    m = a > m ? a : m;
  }
  part[(size_t)blockIdx.y * K + k] = m;
}

__global__ __launch_bounds__(256) void amax_final_kernel(const uint32_t* __restrict__ part, int parts, int K,
                                                         float* __restrict__ amax) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  uint32_t m = 0;
  for (int p = 0; p < parts; ++p) {
    const uint32_t a = part[(size_t)p * K + k];
    m = a > m ? a : m;
  }
  amax[k] = __uint_as_float(m);
}

// Reference output Y = X W in fp32 (X bf16 [M, K], W fp32 [K, N], row-major).
// 64 x 64 tiles, 256 threads with 4 x 4 outputs each, K in chunks of 32
// staged through LDS.  K % 32 == 0; rows and columns past M, N are masked.
__global__ __launch_bounds__(256) void ref_gemm_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                       float* __restrict__ y, int M, int K, int N) {
  __shared__ float xs[32][64 + 4];
  __shared__ float wsm[32][64 + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 32) {
    for (int i = tid; i < 64 * 32; i += 256) {
      const int r = i >> 5, c = i & 31;                 // X: row r, k c
      const int m = m0 + r;
      xs[c][r] = m < M ? __uint_as_float((uint32_t)x[(size_t)m * K + k0 + c] << 16) : 0.0f;
      const int kr = i >> 6, nc = i & 63;               // W: k kr, column nc
      const int n = n0 + nc;
      wsm[kr][nc] = n < N ? w[(size_t)(k0 + kr) * N + n] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], b[4];
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
      for (int j = 0; j < 4; ++j) b[j] = wsm[kk][tx * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) y[(size_t)m * N + n] = acc[i][j];
    }
  }
}

// part[block] = sum over its grid-stride share of (bf16 y - ref)^2, or of
// ref^2 when y is null; fp64 accumulation.
__global__ __launch_bounds__(256) void sqdiff_kernel(const uint16_t* __restrict__ y, const float* __restrict__ ref,
                                                     int64_t n, double* __restrict__ part) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const double r = ref[i];
    const double d = y ? (double)__uint_as_float((uint32_t)y[i] << 16) - r : r;
    s += d * d;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// Device workspace of the search, regions 256-byte aligned.
struct SearchLayout {
  size_t w32, yref, y, sinv, wq, ws, l1k, l2k, fws, fws_bytes, amax, apart, part, total;
};

static bool search_layout(int32_t M, int32_t K, int32_t N, int32_t rank, int32_t fmt, SearchLayout* L) {
  Geometry g;
  if (M < 1 || M > (1 << 20) || !geometry(K, N, rank, fmt, &g)) return false;
  const size_t fws = svdq_workspace_bytes(M, K, rank, fmt);
  if (fws == 0) return false;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
  L->w32 = take((size_t)K * N * 4);
  L->yref = take((size_t)M * N * 4);
  L->y = take((size_t)M * N * 2);
  L->sinv = take((size_t)K * 4);
  L->wq = take(g.wq_bytes);
  L->ws = take(g.ws_bytes);
  L->l1k = take(std::max<size_t>(g.l1k_bytes, 16));
  L->l2k = take(std::max<size_t>(g.l2k_bytes, 16));
  L->fws = take(fws);
  L->fws_bytes = fws;
  L->amax = take((size_t)K * 4);
  L->apart = take((size_t)((M + AMAX_ROWS - 1) / AMAX_ROWS) * K * 4);
  L->part = take((size_t)SR_BLOCKS * 8);
  L->total = o;
  return true;
}

static double sum_parts(const std::vector<double>& p) {
  double s = 0.0;
  for (double v : p) s += v;
  return s;
}

}  // namespace svdq

using namespace svdq;

extern "C" {

int32_t svdq_smooth_candidates(int32_t grids, double* alpha, double* beta) {
  if (grids < 2 || grids > 1000) return 0;
  const int32_t n = 2 * grids - 1;
  if (alpha && beta) {
    alpha[0] = 0.0;
    beta[0] = 0.0;
    for (int32_t a = 1; a < grids; ++a) {
      alpha[a] = (double)a / grids;
      beta[a] = 0.0;
      alpha[grids - 1 + a] = (double)a / grids;
      beta[grids - 1 + a] = 1.0 - (double)a / grids;
    }
  }
  return n;
}

size_t svdq_search_workspace_bytes(int32_t M, int32_t K, int32_t N, int32_t rank, int32_t fmt) {
  SearchLayout L;
  return search_layout(M, K, N, rank, fmt, &L) ? L.total : 0;
}

svdq_status svdq_smooth_search(const float* W, int32_t K, int32_t N, int32_t rank, int32_t fmt,
                               const uint16_t* x_cal, int32_t M, const svdq_search_opts* opts, void* ws,
                               size_t ws_bytes, void* stream, svdq_search_result* res, svdq_prepared* best) {
  if (!W || !x_cal || !ws || !res) return SVDQ_ERR_ARG;
  if (!valid_fmt(fmt)) return SVDQ_ERR_UNSUPPORTED;
  if (!valid_kn(K, N) || !valid_rank(rank) || rank > std::min(K, N)) return SVDQ_ERR_SHAPE;
  const int32_t grids = opts && opts->grids ? opts->grids : 20;
  const int32_t count = svdq_smooth_candidates(grids, nullptr, nullptr);
  if (count == 0) return SVDQ_ERR_ARG;
  SearchLayout SL;
  if (!search_layout(M, K, N, rank, fmt, &SL)) return SVDQ_ERR_SHAPE;
  if ((int64_t)M * K > (int64_t)1 << 32 || (int64_t)N * K > (int64_t)1 << 32) return SVDQ_ERR_SHAPE;
  if (((uintptr_t)x_cal & 15u) || ((uintptr_t)ws & 255u)) return SVDQ_ERR_ALIGN;
  if (ws_bytes < SL.total) return SVDQ_ERR_WORKSPACE;
  if (best && (!best->smooth_inv || !best->wq || !best->ws || (rank > 0 && (!best->l1 || !best->l2))))
    return SVDQ_ERR_ARG;
  for (size_t i = 0; i < (size_t)K * N; ++i)
    if (!std::isfinite(W[i])) return SVDQ_ERR_NUMERIC;
  int devno = 0;
  if (hipGetDevice(&devno) != hipSuccess) return SVDQ_ERR_DEVICE;
  svdq_status s = svdq_device_check(devno);
  if (s != SVDQ_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(ws);
  auto dev = [&](size_t off) { return base + off; };
  auto ok = [](hipError_t e) { return e == hipSuccess; };

  // calibration statistic and reference output
  const int parts = (M + AMAX_ROWS - 1) / AMAX_ROWS;
  hipLaunchKernelGGL(amax_part_kernel, dim3((K + 255) / 256, parts), dim3(256), 0, st, x_cal, M, K,
                     reinterpret_cast<uint32_t*>(dev(SL.apart)));
  hipLaunchKernelGGL(amax_final_kernel, dim3((K + 255) / 256), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t*>(dev(SL.apart)), parts, K, reinterpret_cast<float*>(dev(SL.amax)));
  if (!ok(hipMemcpyAsync(dev(SL.w32), W, (size_t)K * N * 4, hipMemcpyHostToDevice, st))) return SVDQ_ERR_DEVICE;
  hipLaunchKernelGGL(ref_gemm_kernel, dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, st, x_cal,
                     reinterpret_cast<const float*>(dev(SL.w32)), reinterpret_cast<float*>(dev(SL.yref)), M, K, N);
  hipLaunchKernelGGL(sqdiff_kernel, dim3(SR_BLOCKS), dim3(256), 0, st, nullptr,
                     reinterpret_cast<const float*>(dev(SL.yref)), (int64_t)M * N, reinterpret_cast<double*>(dev(SL.part)));
  if (!ok(hipGetLastError())) return SVDQ_ERR_DEVICE;
  std::vector<float> amax(K);
  std::vector<double> part(SR_BLOCKS);
  if (!ok(hipMemcpyAsync(amax.data(), dev(SL.amax), (size_t)K * 4, hipMemcpyDeviceToHost, st)) ||
      !ok(hipMemcpyAsync(part.data(), dev(SL.part), SR_BLOCKS * 8, hipMemcpyDeviceToHost, st)) ||
      !ok(hipStreamSynchronize(st)))
    return SVDQ_ERR_DEVICE;
  for (float a : amax)
    if (!std::isfinite(a)) return SVDQ_ERR_NUMERIC;
  const double ref2 = sum_parts(part);
  if (!(ref2 > 0.0) || !std::isfinite(ref2)) return SVDQ_ERR_NUMERIC;

  // host buffers of one candidate (canonical and kernel layout)
  Geometry g;
  geometry(K, N, rank, fmt, &g);
  std::vector<float> lam(K), sinv(K);
  std::vector<uint16_t> l1((size_t)K * std::max(rank, 1)), l2((size_t)std::max(rank, 1) * N);
  std::vector<uint8_t> wq(canon_code_bytes(N, K, fmt)), wsc(canon_scale_bytes(N, K, fmt));
  std::vector<uint8_t> wq_k(g.wq_bytes), ws_k(g.ws_bytes);
  std::vector<uint16_t> l1k(std::max<size_t>(g.l1k_bytes / 2, 8)), l2k(std::max<size_t>(g.l2k_bytes / 2, 8));
  std::vector<double> alphas(count), betas(count), errs(count, std::nan(""));
  svdq_smooth_candidates(grids, alphas.data(), betas.data());
  svdq_layer layer{K, N, rank, fmt, reinterpret_cast<const float*>(dev(SL.sinv)), dev(SL.wq), dev(SL.ws),
                   reinterpret_cast<const uint16_t*>(dev(SL.l1k)), reinterpret_cast<const uint16_t*>(dev(SL.l2k)),
                   nullptr};
  // Scorer of one prepared candidate (a residual iteration of one (alpha,
  // beta) pair): kernel layout, upload, the fused forward on the
  // calibration rows, and the relative output error against X W.
  Scorer scorer = [&](const CandidateView& v, double* score) -> svdq_status {
    svdq_status ls = svdq_kernel_layout(K, N, rank, fmt, v.smooth_inv, v.wq, v.ws, v.l1b, v.l2b, wq_k.data(),
                                        ws_k.data(), l1k.data(), l2k.data());
    if (ls != SVDQ_OK) return ls;
    if (!ok(hipMemcpyAsync(dev(SL.sinv), v.smooth_inv, (size_t)K * 4, hipMemcpyHostToDevice, st)) ||
        !ok(hipMemcpyAsync(dev(SL.wq), wq_k.data(), g.wq_bytes, hipMemcpyHostToDevice, st)) ||
        !ok(hipMemcpyAsync(dev(SL.ws), ws_k.data(), g.ws_bytes, hipMemcpyHostToDevice, st)) ||
        (rank > 0 && (!ok(hipMemcpyAsync(dev(SL.l1k), l1k.data(), g.l1k_bytes, hipMemcpyHostToDevice, st)) ||
                      !ok(hipMemcpyAsync(dev(SL.l2k), l2k.data(), g.l2k_bytes, hipMemcpyHostToDevice, st)))))
      return SVDQ_ERR_DEVICE;
    ls = svdq_linear_forward(&layer, x_cal, M, reinterpret_cast<uint16_t*>(dev(SL.y)), dev(SL.fws), SL.fws_bytes,
                             stream);
    if (ls != SVDQ_OK) return ls;
    hipLaunchKernelGGL(sqdiff_kernel, dim3(SR_BLOCKS), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(dev(SL.y)), reinterpret_cast<const float*>(dev(SL.yref)),
                       (int64_t)M * N, reinterpret_cast<double*>(dev(SL.part)));
    if (!ok(hipGetLastError()) ||
        !ok(hipMemcpyAsync(part.data(), dev(SL.part), SR_BLOCKS * 8, hipMemcpyDeviceToHost, st)) ||
        !ok(hipStreamSynchronize(st)))
      return SVDQ_ERR_DEVICE;
    *score = std::sqrt(sum_parts(part) / ref2);
    return SVDQ_OK;
  };
  const int32_t iters = opts ? std::max(1, opts->residual_iters) : 1;
  if (iters > SVDQ_MAX_RESIDUAL_ITERS) return SVDQ_ERR_ARG;
  std::vector<double> iter_scores(iters);
  int32_t best_i = -1, best_iter = 0, kept_iter = 0;
  for (int32_t c = 0; c < count; ++c) {
    svdq_prepare_opts po{};
    po.threads = opts ? opts->threads : 0;
    po.residual_iters = iters;
    po.residual_early_stop = opts ? opts->residual_early_stop : 0;
    po.has_beta = 1;
    po.beta = betas[c];
    svdq_prepared pr{};
    pr.lambda = lam.data();
    pr.smooth_inv = sinv.data();
    pr.l1 = rank ? l1.data() : nullptr;
    pr.l2 = rank ? l2.data() : nullptr;
    pr.wq = wq.data();
    pr.ws = wsc.data();
    pr.iter_errors = iter_scores.data();
    pr.best_iter = &kept_iter;
    // each residual iteration is scored by the calibration output error
    // (AutoRound doc, "Residual iteration": output error when smooth is on)
    s = prepare_layer(W, amax.data(), K, N, alphas[c], rank, fmt, &po, &pr, &scorer);
    if (s == SVDQ_ERR_NUMERIC) continue;          // a candidate lambda out of range scores NaN
    if (s != SVDQ_OK) return s;
    errs[c] = iter_scores[kept_iter];
    if (std::isfinite(errs[c]) && (best_i < 0 || errs[c] < errs[best_i])) {
      best_i = c;
      best_iter = kept_iter;
      if (best) {
        std::memcpy(best->smooth_inv, sinv.data(), (size_t)K * 4);
        if (best->lambda) std::memcpy(best->lambda, lam.data(), (size_t)K * 4);
        std::memcpy(best->wq, wq.data(), wq.size());
        std::memcpy(best->ws, wsc.data(), wsc.size());
        if (rank > 0) {
          std::memcpy(best->l1, l1.data(), (size_t)K * rank * 2);
          std::memcpy(best->l2, l2.data(), (size_t)rank * N * 2);
        }
      }
    }
  }
  res->count = count;
  res->best = best_i;
  res->best_iter = best_i < 0 ? -1 : best_iter;
  if (res->errors)
    for (int32_t c = 0; c < count; ++c) res->errors[c] = errs[c];
  if (best_i < 0) return SVDQ_ERR_NUMERIC;
  res->alpha = alphas[best_i];
  res->beta = betas[best_i];
  return SVDQ_OK;
}

}  // extern "C"
