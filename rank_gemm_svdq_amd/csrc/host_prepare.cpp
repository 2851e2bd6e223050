// Host side of the C ABI: argument checks, sizes and layouts, calibration
// statistics, RTN packers, the offline prepare, LoRA attach, kernel-layout
// conversion and the workspace read-back helper.
//
// Compiled without fp contraction: the packers must reproduce IEEE fp32
// products and divisions exactly (the quantized codes and scales are
// specified bit for bit).

#include <sched.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "host_internal.h"

namespace svdq {

// ---------------------------------------------------------------- shapes

bool valid_kn(int32_t K, int32_t N) {
  return K >= kStep && K <= 65536 && K % kStep == 0 && N >= 16 && N <= 262144 && N % 16 == 0;
}
bool valid_rank(int32_t rank) { return rank >= 0 && rank <= SVDQ_MAX_RANK && rank % 16 == 0; }
bool valid_fmt(int32_t fmt) { return fmt == SVDQ_INT4_G64 || is_mx(fmt) || fmt == SVDQ_W8A8; }

bool geometry(int32_t K, int32_t N, int32_t rank, int32_t fmt, Geometry* g) {
  if (!valid_kn(K, N) || !valid_rank(rank) || !valid_fmt(fmt)) return false;
  g->K = K; g->N = N; g->rank = rank; g->rpad = rank_pad(rank); g->fmt = fmt;
  g->steps = K / kStep;
  g->ks4 = (g->steps + 3) / 4;
  g->csteps = code_steps(K, fmt);
  g->wq_bytes = code_bytes(N, g->csteps);   // N % 16 == 0: exactly the canonical size
  g->wq_tail_off = g->wq_bytes;
  if (fmt == SVDQ_INT4_G64) g->wq_bytes += i4_tail_bytes(N, g->steps);   // FP6 codes: main parts, then tails
  g->ws_bytes = fmt == SVDQ_INT4_G64   ? i4_scale_bytes(N, g->steps)
                : is_mx(fmt)            ? scale_record_bytes(N, g->ks4)
                                        : (size_t)N * 4;
  g->l1k_bytes = (size_t)K * rank * 2;
  g->l2k_bytes = (size_t)N * g->rpad * 2;
  return true;
}

int32_t choose_zsplit(int32_t, int32_t) { return 1; }   // K-A reduces Z inside each block

// 0 requested: OMP_NUM_THREADS when set, else the CPUs this process may run
// on; at most 64.
int default_threads(int requested) {
  if (requested > 0) return requested;
  if (const char* env = std::getenv("OMP_NUM_THREADS")) {
    const long v = std::strtol(env, nullptr, 10);
    if (v > 0) return (int)std::min(v, 64L);
  }
  cpu_set_t set;
  CPU_ZERO(&set);
  int h = sched_getaffinity(0, sizeof(set), &set) == 0 ? CPU_COUNT(&set) : 0;
  if (h <= 0) h = (int)std::thread::hardware_concurrency();
  return h > 0 ? std::min(h, 64) : 1;
}

// ----------------------------------------------------------- conversions

uint16_t bf16_from_double(double x) {
  uint64_t b;
  std::memcpy(&b, &x, 8);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000);
  const int ex = (int)((b >> 52) & 0x7FF);
  const uint64_t man = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return sign | (man ? 0x7FC0 : 0x7F80);
  if (ex == 0) return sign;                       // binary64 subnormals are far below bf16's range
  int e = ex - 1023;
  if (e >= -126) {                                // normal bf16: keep 7 fraction bits
    uint64_t keep = man >> 45, rest = man & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    if (rest > half || (rest == half && (keep & 1))) ++keep;
    if (keep == 128) { keep = 0; ++e; }
    if (e > 127) return sign | 0x7F80;
    return sign | (uint16_t)((e + 127) << 7) | (uint16_t)keep;
  }
  // subnormal bf16: multiples of 2^-133; x = full * 2^(e-52)
  const int sh = -81 - e;                         // q = full / 2^sh, sh >= 46
  if (sh >= 64) return sign;
  const uint64_t full = man | (1ull << 52);
  uint64_t q = full >> sh, rest = full & ((1ull << sh) - 1);
  const uint64_t half = 1ull << (sh - 1);
  if (rest > half || (rest == half && (q & 1))) ++q;
  return sign | (uint16_t)q;                      // q == 128 is the smallest normal
}

double double_from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

uint16_t half_from_float(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint16_t sign = (uint16_t)((x >> 16) & 0x8000);
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return sign | 0x7C00 | (ax > 0x7F800000u ? 0x200 : 0);
  const int e = (int)(ax >> 23) - 127;
  const uint32_t m = ax & 0x7FFFFFu;
  if (e >= -14) {
    uint32_t h = ((uint32_t)(e + 15) << 10) | (m >> 13);
    const uint32_t rest = m & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1))) ++h;   // may carry into the exponent
    if (h >= 0x7C00u) return sign | 0x7C00;
    return sign | (uint16_t)h;
  }
  if (e < -25) return sign;
  // subnormal binary16: q * 2^-24 with q = full * 2^(e+1), full the 24-bit significand
  const uint32_t full = m | 0x800000u;
  const int sh = -(e + 1);                        // 14..24
  uint32_t q = full >> sh, rest = full & ((1u << sh) - 1);
  const uint32_t half = 1u << (sh - 1);
  if (rest > half || (rest == half && (q & 1))) ++q;
  return sign | (uint16_t)q;
}

float float_from_half(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000) << 16;
  const int ex = (h >> 10) & 0x1F;
  const uint32_t m = h & 0x3FF;
  float f;
  if (ex == 0) {
    f = std::ldexp((float)m, -24);
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u |= sign;
    std::memcpy(&f, &u, 4);
    return f;
  }
  uint32_t u = ex == 0x1F ? (sign | 0x7F800000u | (m << 13)) : (sign | ((uint32_t)(ex - 15 + 127) << 23) | (m << 13));
  std::memcpy(&f, &u, 4);
  return f;
}

// ------------------------------------------------------------ quantizers

// INT4 (Zhou notes sec. 2.2 Eq. (1); 64 elements, fp16 scale): s32 = amax/7
// in fp32, s16 = fp16(s32), codes = clamp(rint(x * fp32(1/s16)), -7, 7).  A
// scale past the fp16 range saturates at 65504 (the largest finite binary16
// value; the clamp then clips the codes) instead of becoming infinite.
void quant_int4_group(const float* x, uint8_t* nib, uint16_t* scale_bits) {
  float amax = 0.0f;
  for (int i = 0; i < 64; ++i) amax = std::max(amax, std::fabs(x[i]));
  const float s32 = amax / 7.0f;
  uint16_t s16 = half_from_float(s32);
  if (s16 == 0x7C00) s16 = 0x7BFF;
  const float sf = float_from_half(s16);
  *scale_bits = s16;
  if (sf == 0.0f) {
    std::memset(nib, 0, 64);
    return;
  }
  const float rcp = 1.0f / sf;
  for (int i = 0; i < 64; ++i) {
    float y = x[i] * rcp;
    float q = std::nearbyint(y);
    q = std::min(7.0f, std::max(-7.0f, q));
    nib[i] = (uint8_t)((int)q & 0xF);
  }
}

// MXFP4 (E2M1, 32 elements, E8M0 scale): e = smallest integer with
// amax <= 6 * 2^e (clamped to [-127, 127]), or with the OCP rule
// e = floor(log2(amax)) - 2; code = nearest E2M1 magnitude of |x| 2^-e with
// ties to the even mantissa, saturated at 6 (only the OCP rule reaches it);
// bit 3 = sign of x.
void quant_mxfp4_group(const float* x, uint8_t* nib, uint8_t* scale_byte, bool ocp_rule) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(x[i]));
  int e;
  if (amax == 0.0f) {
    e = -127;
  } else {
    int E;
    const float f = std::frexp(amax, &E);   // amax = f 2^E, 0.5 <= f < 1
    e = ocp_rule ? E - 3 : (f <= 0.75f ? E - 3 : E - 2);
    e = std::min(127, std::max(-127, e));
  }
  *scale_byte = (uint8_t)(e + 127);
  const double inv = std::ldexp(1.0, -e);
  for (int i = 0; i < 32; ++i) {
    const double a = std::fabs((double)x[i]) * inv;
    const int c = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0);
    nib[i] = (uint8_t)(c | (std::signbit(x[i]) ? 8 : 0));
  }
}

// 8-bit (one fp32 scale per row of K values): s = fp32(amax / 127),
// codes = clamp(rint(x * fp32(1/s)), -127, 127), zero elements 0; s == 0
// gives all zeros.
void quant_w8_row(const float* x, int32_t K, int8_t* q, float* scale) {
  float amax = 0.0f;
  for (int32_t i = 0; i < K; ++i) amax = std::max(amax, std::fabs(x[i]));
  const float s = amax / 127.0f;
  *scale = s;
  if (s == 0.0f) {
    std::memset(q, 0, (size_t)K);
    return;
  }
  const float rcp = 1.0f / s;   // infinite when s is below 2^-128: zeros stay 0
  for (int32_t i = 0; i < K; ++i) {
    float v = x[i] == 0.0f ? 0.0f : std::nearbyint(x[i] * rcp);
    v = std::min(127.0f, std::max(-127.0f, v));
    q[i] = (int8_t)v;
  }
}

static bool all_finite(const float* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

}  // namespace svdq

using namespace svdq;

// ============================================================== C ABI

extern "C" {

const char* svdq_status_str(svdq_status s) {
  switch (s) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_ARG: return "invalid argument";
    case SVDQ_ERR_SHAPE: return "unsupported shape";
    case SVDQ_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case SVDQ_ERR_UNSUPPORTED: return "unsupported format or device";
    case SVDQ_ERR_WORKSPACE: return "workspace too small";
    case SVDQ_ERR_NUMERIC: return "non-finite input or solver failure";
    case SVDQ_ERR_DEVICE: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t svdq_abi_version(void) { return SVDQ_ABI_VERSION; }

svdq_status svdq_layer_sizes(int32_t K, int32_t N, int32_t rank, int32_t fmt, svdq_sizes* out) {
  if (!out) return SVDQ_ERR_ARG;
  if (!valid_fmt(fmt)) return SVDQ_ERR_UNSUPPORTED;
  Geometry g;
  if (!geometry(K, N, rank, fmt, &g)) return SVDQ_ERR_SHAPE;
  out->wq_bytes = g.wq_bytes;
  out->ws_bytes = g.ws_bytes;
  out->l1k_bytes = g.l1k_bytes;
  out->l2k_bytes = g.l2k_bytes;
  out->wq_canon_bytes = canon_code_bytes(N, K, fmt);
  out->ws_canon_bytes = canon_scale_bytes(N, K, fmt);
  return SVDQ_OK;
}

svdq_status svdq_workspace_layout(int32_t M, int32_t K, int32_t rank, int32_t fmt, svdq_ws_layout* out) {
  if (!out) return SVDQ_ERR_ARG;
  if (!valid_fmt(fmt)) return SVDQ_ERR_UNSUPPORTED;
  if (M < 1 || M > (1 << 20) || !valid_kn(K, 16) || !valid_rank(rank)) return SVDQ_ERR_SHAPE;
  const int32_t steps = K / kStep, ks4 = (steps + 3) / 4;
  out->zsplit = rank > 0 ? choose_zsplit(M, K) : 0;
  out->xq_off = 0;
  out->xq_bytes = code_bytes(M, code_steps(K, fmt));
  if (fmt == SVDQ_INT4_G64) out->xq_bytes += i4_tail_bytes(M, steps);   // main parts, then tails
  out->xs_off = align256(out->xq_bytes);
  out->xs_bytes = is_w8(fmt)                ? (size_t)(M + 15) / 16 * 64
                  : fmt == SVDQ_INT4_G64 ? i4_scale_bytes(M, steps)
                                            : scale_record_bytes(M, ks4);
  out->z_off = align256(out->xs_off + out->xs_bytes);
  out->z_bytes = rank > 0 ? (size_t)out->zsplit * M * rank_pad(rank) * 4 : 0;
  out->total = align256(out->z_off + out->z_bytes);
  return SVDQ_OK;
}

size_t svdq_workspace_bytes(int32_t M, int32_t K, int32_t rank, int32_t fmt) {
  svdq_ws_layout l;
  return svdq_workspace_layout(M, K, rank, fmt, &l) == SVDQ_OK ? l.total : 0;
}

svdq_status svdq_calib_absmax(const uint16_t* x, int64_t rows, int32_t K, float* amax) {
  if (!x || !amax || rows < 0 || K <= 0) return SVDQ_ERR_ARG;
  for (int64_t i = 0; i < rows; ++i) {
    const uint16_t* row = x + i * K;
    for (int32_t k = 0; k < K; ++k) {
      const uint16_t h = row[k];
      if ((h & 0x7F80) == 0x7F80) return SVDQ_ERR_NUMERIC;
      const float a = (float)std::fabs(double_from_bf16(h));
      if (a > amax[k]) amax[k] = a;
    }
  }
  return SVDQ_OK;
}

svdq_status svdq_pack_host(const float* x, int32_t rows, int32_t K, int32_t fmt, uint8_t* codes, uint8_t* scales) {
  if (!x || !codes || !scales || rows < 0) return SVDQ_ERR_ARG;
  if (!valid_fmt(fmt)) return SVDQ_ERR_UNSUPPORTED;
  if (is_w8(fmt)) {
    if (K <= 0) return SVDQ_ERR_SHAPE;
    parallel_for(rows, default_threads(0), [&](int64_t lo, int64_t hi) {
      for (int64_t r = lo; r < hi; ++r) {
        float sc;
        quant_w8_row(x + (size_t)r * K, K, reinterpret_cast<int8_t*>(codes) + (size_t)r * K, &sc);
        std::memcpy(scales + (size_t)r * 4, &sc, 4);
      }
    });
    return SVDQ_OK;
  }
  const int G = group_size(fmt);
  if (K <= 0 || K % G != 0) return SVDQ_ERR_SHAPE;
  parallel_for(rows, default_threads(0), [&](int64_t lo, int64_t hi) {
    uint8_t nib[64];
    for (int64_t r = lo; r < hi; ++r) {
      for (int32_t g = 0; g < K / G; ++g) {
        const float* src = x + (size_t)r * K + (size_t)g * G;
        if (fmt == SVDQ_INT4_G64) {
          uint16_t sb;
          quant_int4_group(src, nib, &sb);
          std::memcpy(scales + ((size_t)r * (K / 64) + g) * 2, &sb, 2);
        } else {
          quant_mxfp4_group(src, nib, scales + (size_t)r * (K / 32) + g, fmt == SVDQ_MXFP4_G32_OCP);
        }
        uint8_t* dst = codes + (size_t)r * (K / 2) + (size_t)g * (G / 2);
        for (int i = 0; i < G / 2; ++i) dst[i] = (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));
      }
    }
  });
  return SVDQ_OK;
}

svdq_status svdq_attach_lora(const float* lambda, const uint16_t* l1, const uint16_t* l2, int32_t K, int32_t N,
                             int32_t rank, const float* A, const float* B, int32_t k, float strength,
                             uint16_t* l1_out, uint16_t* l2_out) {
  if (!lambda || !A || !B || !l1_out || !l2_out || (rank > 0 && (!l1 || !l2))) return SVDQ_ERR_ARG;
  if (!valid_kn(K, N) || !valid_rank(rank) || k < 0 || k % 16 || rank + k > SVDQ_MAX_RANK) return SVDQ_ERR_SHAPE;
  const int32_t rt = rank + k;
  for (int32_t i = 0; i < K; ++i) {
    for (int32_t j = 0; j < rank; ++j) l1_out[(size_t)i * rt + j] = l1[(size_t)i * rank + j];
    for (int32_t j = 0; j < k; ++j)
      l1_out[(size_t)i * rt + rank + j] = bf16_from_double((double)lambda[i] * (double)A[(size_t)i * k + j]);
  }
  for (int32_t j = 0; j < rank; ++j)
    std::memcpy(l2_out + (size_t)j * N, l2 + (size_t)j * N, sizeof(uint16_t) * N);
  for (int32_t j = 0; j < k; ++j)
    for (int32_t n = 0; n < N; ++n)
      l2_out[(size_t)(rank + j) * N + n] = bf16_from_double((double)strength * (double)B[(size_t)j * N + n]);
  return SVDQ_OK;
}

// Value of canonical code `nib` under its group's scale (exact in fp64).
static double decode_int4(uint8_t nib, uint16_t s16) {
  const int q = (nib & 8) ? (int)nib - 16 : (int)nib;
  return (double)q * (double)float_from_half(s16);
}
static double decode_mxfp4(uint8_t nib, uint8_t e8m0) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const double v = std::ldexp(mag[nib & 7], (int)e8m0 - 127);
  return (nib & 8) ? -v : v;
}

// Canonical codes [N, K/2] + scales -> decoded values transposed to [K, N].
static void decode_transposed(const uint8_t* wq, const uint8_t* ws, int32_t N, int32_t K, int32_t fmt, int threads,
                              double* out) {
  constexpr int32_t NB = 32;
  const int32_t G = is_w8(fmt) ? K : group_size(fmt);
  parallel_for((N + NB - 1) / NB, threads, [&](int64_t lo, int64_t hi) {
    std::vector<double> blk((size_t)NB * K);
    for (int64_t b = lo; b < hi; ++b) {
      const int32_t n0 = (int32_t)b * NB, nn = std::min(NB, N - n0);
      for (int32_t i = 0; i < nn; ++i) {
        const int32_t n = n0 + i;
        if (is_w8(fmt)) {
          float sc;
          std::memcpy(&sc, ws + 4 * (size_t)n, 4);
          const int8_t* q8 = reinterpret_cast<const int8_t*>(wq) + (size_t)n * K;
          for (int32_t k = 0; k < K; ++k) blk[(size_t)i * K + k] = (double)q8[k] * (double)sc;
          continue;
        }
        const uint8_t* codes = wq + (size_t)n * (K / 2);
        for (int32_t k = 0; k < K; ++k) {
          const uint8_t nib = (codes[k >> 1] >> ((k & 1) * 4)) & 0xF;
          const size_t g = (size_t)n * (K / G) + k / G;
          double v;
          if (fmt == SVDQ_INT4_G64) {
            uint16_t s16;
            std::memcpy(&s16, ws + 2 * g, 2);
            v = decode_int4(nib, s16);
          } else {
            v = decode_mxfp4(nib, ws[g]);
          }
          blk[(size_t)i * K + k] = v;
        }
      }
      for (int32_t k = 0; k < K; ++k)
        for (int32_t i = 0; i < nn; ++i) out[(size_t)k * N + n0 + i] = blk[(size_t)i * K + k];
    }
  });
}

// One candidate of the residual iteration: bf16 factors of the top-r split
// of `target`, R = W~ - L1b L2b (fp64, kept), its RTN codes and the error
// ||W~ - L1b L2b - Q(R)||_F.
struct Candidate {
  std::vector<uint16_t> l1b, l2b;
  std::vector<double> sig, r64, qr;  // qr: Q(R) in [K, N]
  std::vector<uint8_t> wq, ws;
  double err = 0.0;
  int32_t iter = 0;
};

static svdq_status fit_candidate(const std::vector<double>& wt, const double* target, int32_t K, int32_t N,
                                 int32_t rank, int32_t fmt, int threads, int max_iters, Candidate& c) {
  std::vector<double> L1, L2;
  if (!truncated_svd(target, K, N, rank, threads, max_iters, L1, L2, c.sig)) return SVDQ_ERR_NUMERIC;
  c.l1b.resize((size_t)K * rank);
  c.l2b.resize((size_t)rank * N);
  std::vector<double> l1d(c.l1b.size()), l2d(c.l2b.size());
  for (size_t i = 0; i < l1d.size(); ++i) { c.l1b[i] = bf16_from_double(L1[i]); l1d[i] = double_from_bf16(c.l1b[i]); }
  for (size_t i = 0; i < l2d.size(); ++i) { c.l2b[i] = bf16_from_double(L2[i]); l2d[i] = double_from_bf16(c.l2b[i]); }
  // R = W~ - L1b L2b in fp64; its fp32 transpose feeds the packer
  c.r64.resize((size_t)K * N);
  std::vector<float> rt((size_t)N * K);
  parallel_for(K, threads, [&](int64_t lo, int64_t hi) {
    std::vector<double> acc(N);
    for (int64_t i = lo; i < hi; ++i) {
      for (int32_t j = 0; j < N; ++j) acc[j] = 0.0;
      for (int32_t p = 0; p < rank; ++p) {
        const double a = l1d[(size_t)i * rank + p];
        const double* b = &l2d[(size_t)p * N];
        for (int32_t j = 0; j < N; ++j) acc[j] += a * b[j];
      }
      for (int32_t j = 0; j < N; ++j) {
        const double r = wt[(size_t)i * N + j] - acc[j];
        c.r64[(size_t)i * N + j] = r;
        rt[(size_t)j * K + i] = (float)r;
      }
    }
  });
  c.wq.resize(canon_code_bytes(N, K, fmt));
  c.ws.resize(canon_scale_bytes(N, K, fmt));
  const svdq_status st = svdq_pack_host(rt.data(), N, K, fmt, c.wq.data(), c.ws.data());
  if (st != SVDQ_OK) return st;
  // Q(R) = decoded codes, transposed back to [K, N]; error = ||R - Q(R)||_F
  c.qr.resize((size_t)K * N);
  decode_transposed(c.wq.data(), c.ws.data(), N, K, fmt, threads, c.qr.data());
  std::vector<double> rowerr(K);
  parallel_for(K, threads, [&](int64_t lo, int64_t hi) {
    for (int64_t k = lo; k < hi; ++k) {
      double e = 0.0;
      for (int32_t n = 0; n < N; ++n) {
        const double d = c.r64[(size_t)k * N + n] - c.qr[(size_t)k * N + n];
        e += d * d;
      }
      rowerr[k] = e;
    }
  });
  double e = 0.0;
  for (double v : rowerr) e += v;
  c.err = std::sqrt(e);
  return SVDQ_OK;
}

}  // extern "C"

namespace svdq {

// The offline preparation; `scorer` (optional) replaces the weight
// reconstruction error as the residual iterations' score.
svdq_status prepare_layer(const float* W, const float* act_amax, int32_t K, int32_t N, double alpha, int32_t rank,
                          int32_t fmt, const svdq_prepare_opts* opts, svdq_prepared* out, const Scorer* scorer) {
  if (!W || !act_amax || !out || !out->smooth_inv || !out->wq || !out->ws) return SVDQ_ERR_ARG;
  if (!valid_fmt(fmt)) return SVDQ_ERR_UNSUPPORTED;
  if (!valid_kn(K, N) || !valid_rank(rank) || rank > std::min(K, N)) return SVDQ_ERR_SHAPE;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return SVDQ_ERR_ARG;
  const int32_t lk = opts ? opts->lora_rank : 0;
  if (lk < 0 || lk % 16 || rank + lk > SVDQ_MAX_RANK) return SVDQ_ERR_SHAPE;
  if (lk > 0 && (!opts->lora_a || !opts->lora_b)) return SVDQ_ERR_ARG;
  if (rank + lk > 0 && (!out->l1 || !out->l2)) return SVDQ_ERR_ARG;
  if (rank > 0 && std::min(K, N) > 16384) return SVDQ_ERR_SHAPE;
  const int32_t iters = opts ? std::max(1, opts->residual_iters) : 1;
  if (iters > SVDQ_MAX_RESIDUAL_ITERS) return SVDQ_ERR_ARG;
  const bool early_stop = opts && opts->residual_early_stop;
  const double beta = (opts && opts->has_beta) ? opts->beta : 1.0 - alpha;
  if (!(beta >= 0.0 && beta <= 1.0)) return SVDQ_ERR_ARG;
  const int threads = default_threads(opts ? opts->threads : 0);
  const int max_iters = opts ? opts->max_iters : 0;
  if (!all_finite(W, (size_t)K * N) || !all_finite(act_amax, K)) return SVDQ_ERR_NUMERIC;
  for (int32_t i = 0; i < K; ++i)
    if (act_amax[i] < 0.0f) return SVDQ_ERR_ARG;
  if (lk > 0 && (!all_finite(opts->lora_a, (size_t)K * lk) || !all_finite(opts->lora_b, (size_t)lk * N) ||
                 !std::isfinite(opts->lora_strength)))
    return SVDQ_ERR_NUMERIC;

  // lambda (Eq. (4), weight exponent beta); a zero statistic leaves the channel unscaled
  std::vector<float> lam(K), inv(K);
  for (int32_t i = 0; i < K; ++i) {
    float aw = 0.0f;
    const float* row = W + (size_t)i * N;
    for (int32_t j = 0; j < N; ++j) aw = std::max(aw, std::fabs(row[j]));
    const double ax = act_amax[i];
    double l = 1.0;
    if (ax > 0.0 && aw > 0.0f) l = std::pow(ax, alpha) / std::pow((double)aw, beta);
    lam[i] = (float)l;
    if (!std::isfinite(lam[i]) || lam[i] == 0.0f) return SVDQ_ERR_NUMERIC;
    inv[i] = 1.0f / lam[i];
  }
  // W~ = diag(lambda) W (exact in fp64)
  std::vector<double> wt((size_t)K * N);
  parallel_for(K, threads, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i)
      for (int32_t j = 0; j < N; ++j) wt[(size_t)i * N + j] = (double)lam[i] * (double)W[(size_t)i * N + j];
  });
  // residual iteration: candidate t fits W~ (t = 0) or W~ - Q(R_{t-1})
  Candidate best, cur;
  std::vector<double> target;
  if (out->iter_errors)
    for (int32_t t = 0; t < iters; ++t) out->iter_errors[t] = std::nan("");
  for (int32_t t = 0; t < iters; ++t) {
    const svdq_status st = fit_candidate(wt, t == 0 ? wt.data() : target.data(), K, N, rank, fmt, threads,
                                         max_iters, cur);
    if (st != SVDQ_OK) return st;
    cur.iter = t;
    if (scorer) {
      const CandidateView v{lam.data(), inv.data(), rank ? cur.l1b.data() : nullptr, rank ? cur.l2b.data() : nullptr,
                            cur.wq.data(), cur.ws.data()};
      const svdq_status ss = (*scorer)(v, &cur.err);
      if (ss != SVDQ_OK) return ss;
    }
    if (out->iter_errors) out->iter_errors[t] = cur.err;
    if (t + 1 < iters) {
      target.resize((size_t)K * N);
      parallel_for(K, threads, [&](int64_t lo, int64_t hi) {
        for (size_t i = (size_t)lo * N; i < (size_t)hi * N; ++i) target[i] = wt[i] - cur.qr[i];
      });
    }
    // the smallest score wins, the earlier on ties; a non-finite score
    // never displaces a finite one
    if (t == 0 || cur.err < best.err || (!std::isfinite(best.err) && std::isfinite(cur.err))) {
      std::swap(best, cur);
    } else if (early_stop && cur.err > best.err) {
      break;
    }
  }
  std::memcpy(out->wq, best.wq.data(), best.wq.size());
  std::memcpy(out->ws, best.ws.data(), best.ws.size());
  if (out->residual)
    for (size_t i = 0; i < best.r64.size(); ++i) out->residual[i] = (float)best.r64[i];
  if (out->best_iter) *out->best_iter = best.iter;
  for (int32_t i = 0; i < K; ++i) {
    out->smooth_inv[i] = inv[i];
    if (out->lambda) out->lambda[i] = lam[i];
  }
  if (out->sigma)
    for (int32_t j = 0; j < rank; ++j) out->sigma[j] = best.sig[j];
  if (rank + lk > 0) {
    if (lk > 0) {
      const svdq_status st = svdq_attach_lora(lam.data(), best.l1b.data(), best.l2b.data(), K, N, rank,
                                              opts->lora_a, opts->lora_b, lk, opts->lora_strength, out->l1, out->l2);
      if (st != SVDQ_OK) return st;
    } else {
      std::memcpy(out->l1, best.l1b.data(), best.l1b.size() * 2);
      std::memcpy(out->l2, best.l2b.data(), best.l2b.size() * 2);
    }
  }
  return SVDQ_OK;
}

}  // namespace svdq

extern "C" {

svdq_status svdq_prepare(const float* W, const float* act_amax, int32_t K, int32_t N, double alpha, int32_t rank,
                         int32_t fmt, const svdq_prepare_opts* opts, svdq_prepared* out) {
  return prepare_layer(W, act_amax, K, N, alpha, rank, fmt, opts, out, nullptr);
}

int64_t svdq_reservoir_select(int64_t n_calls, int64_t k, uint64_t seed, int64_t* out) {
  if (!out) return -1;
  if (n_calls <= 0 || k <= 0) return 0;
  const int64_t kept = std::min(n_calls, k);
  for (int64_t i = 0; i < kept; ++i) out[i] = i;
  uint64_t state = seed;
  for (int64_t i = k; i < n_calls; ++i) {
    // SplitMix64
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    const uint64_t j = (uint64_t)(((unsigned __int128)z * (unsigned __int128)(uint64_t)(i + 1)) >> 64);
    if (j < (uint64_t)k) out[j] = i;
  }
  std::sort(out, out + kept);
  return kept;
}

svdq_status svdq_kernel_layout(int32_t K, int32_t N, int32_t rank, int32_t fmt, const float* smooth_inv,
                               const uint8_t* wq, const uint8_t* ws, const uint16_t* l1, const uint16_t* l2,
                               uint8_t* wq_k, uint8_t* ws_k, uint16_t* l1k, uint16_t* l2k) {
  if (!smooth_inv || !wq || !ws || !wq_k || !ws_k) return SVDQ_ERR_ARG;
  if (!valid_fmt(fmt)) return SVDQ_ERR_UNSUPPORTED;
  Geometry g;
  if (!geometry(K, N, rank, fmt, &g)) return SVDQ_ERR_SHAPE;
  if (rank > 0 && (!l1 || !l2 || !l1k || !l2k)) return SVDQ_ERR_ARG;
  const int32_t steps = g.steps, rp = g.rpad;
  if (is_w8(fmt)) {
    // 8-bit codes: element k of row n is byte k % 64 of 64-byte step k / 64;
    // the per-channel fp32 scales are stored as they are
    const int32_t cs = g.csteps;
    parallel_for(N, default_threads(0), [&](int64_t lo, int64_t hi) {
      for (int64_t n = lo; n < hi; ++n)
        for (int32_t k = 0; k < K; ++k) wq_k[code_offset((int)n, k >> 6, k & 63, cs)] = wq[(size_t)n * K + k];
    });
    std::memcpy(ws_k, ws, (size_t)N * 4);
  } else if (is_mx(fmt)) {
    // codes: tiled 1 KB units
    parallel_for(N, default_threads(0), [&](int64_t lo, int64_t hi) {
      for (int64_t n = lo; n < hi; ++n)
        for (int32_t t = 0; t < steps; ++t) {
          const uint8_t* src = wq + (size_t)n * (K / 2) + (size_t)t * 64;
          for (int b = 0; b < 64; ++b) wq_k[code_offset((int)n, t, b, steps)] = src[b];
        }
    });
    // scales
    std::memset(ws_k, 127, g.ws_bytes);
    for (int32_t n = 0; n < N; ++n)
      for (int32_t b = 0; b < K / 32; ++b) {
        const int32_t t = b / 4, gq = b % 4;
        ws_k[scale_record_offset(wrec_row(n), t / 4, 4 * gq + t % 4, g.ks4)] = ws[(size_t)n * (K / 32) + b];
      }
  } else {
    // INT4: FP6 E2M3 codes, per slice dwords 0-3 in the main part and 4-5 in
    // the tail part (padding rows of the last 32-row tail unit stay zero)
    std::memset(wq_k, 0, g.wq_bytes);
    uint8_t* tail = wq_k + g.wq_tail_off;
    parallel_for(N, default_threads(0), [&](int64_t lo, int64_t hi) {
      for (int64_t n = lo; n < hi; ++n)
        for (int32_t t = 0; t < steps; ++t)
          for (int sl = 0; sl < 4; ++sl) {
            uint8_t c[32];
            for (int j = 0; j < 32; ++j) {
              const int32_t k = t * kStep + 32 * sl + j;
              const int nib = (wq[(size_t)n * (K / 2) + k / 2] >> ((k & 1) * 4)) & 0xF;
              c[j] = e2m3_of_int4(nib >= 8 ? nib - 16 : nib);
            }
            uint32_t d[6];
            pack6(c, d);
            std::memcpy(wq_k + i4_main_offset((int)n, t, sl, steps), d, 16);
            std::memcpy(tail + i4_tail_offset((int)n, t, sl, steps), d + 4, 8);
          }
    });
    const uint16_t* s16 = reinterpret_cast<const uint16_t*>(ws);
    std::memset(ws_k, 0, g.ws_bytes);
    for (int32_t n = 0; n < N; ++n)
      for (int32_t t = 0; t < steps; ++t)
        for (int G = 0; G < 2; ++G)
          std::memcpy(ws_k + i4_wscale_offset(n, t, G, steps), s16 + (size_t)n * (K / 64) + 2 * t + G, 2);
  }
  if (rank == 0) return SVDQ_OK;
  // down factor: L1' (bf16) in the order of K-A's MFMA B operand,
  // [step][s 0..3][n-tile][lane 0..63][i 0..7] with
  // k = 128 step + 32 (lane / 16) + 8 s + i and n = 16 tile + lane % 16
  const int32_t ntile = rank / 16;
  parallel_for(steps, default_threads(0), [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t)
      for (int s = 0; s < 4; ++s)
        for (int32_t nt = 0; nt < ntile; ++nt)
          for (int lane = 0; lane < 64; ++lane)
            for (int i = 0; i < 8; ++i) {
              const int32_t k = (int32_t)t * kStep + 32 * (lane / 16) + 8 * s + i;
              const int32_t n = 16 * nt + lane % 16;
              const size_t idx = (((((size_t)t * 4 + s) * ntile + nt) * 64 + lane) * 8) + i;
              l1k[idx] = l1[(size_t)k * rank + n];
            }
  });
  // up factor: L2'^T padded to rpad columns
  for (int32_t n = 0; n < N; ++n)
    for (int32_t j = 0; j < rp; ++j) l2k[(size_t)n * rp + j] = j < rank ? l2[(size_t)j * N + n] : 0;
  return SVDQ_OK;
}

svdq_status svdq_unpack_activations(const void* ws_host, int32_t M, int32_t K, int32_t rank, int32_t fmt,
                                    uint8_t* xq, uint8_t* xs, float* z) {
  if (!ws_host || !xq || !xs) return SVDQ_ERR_ARG;
  svdq_ws_layout L;
  svdq_status st = svdq_workspace_layout(M, K, rank, fmt, &L);
  if (st != SVDQ_OK) return st;
  const uint8_t* base = static_cast<const uint8_t*>(ws_host);
  const uint8_t* q = base + L.xq_off;
  const int32_t steps = K / kStep, ks4 = (steps + 3) / 4;
  if (is_w8(fmt)) {
    const int32_t cs = code_steps(K, fmt);
    for (int32_t m = 0; m < M; ++m)
      for (int32_t k = 0; k < K; ++k) xq[(size_t)m * K + k] = q[code_offset(m, k >> 6, k & 63, cs)];
    std::memcpy(xs, base + L.xs_off, (size_t)M * 4);
  } else if (is_mx(fmt)) {
    for (int32_t m = 0; m < M; ++m)
      for (int32_t t = 0; t < steps; ++t)
        for (int b = 0; b < 64; ++b) xq[(size_t)m * (K / 2) + (size_t)t * 64 + b] = q[code_offset(m, t, b, steps)];
    const uint8_t* s = base + L.xs_off;
    for (int32_t m = 0; m < M; ++m)
      for (int32_t b = 0; b < K / 32; ++b) {
        const int32_t t = b / 4, gq = b % 4;
        xs[(size_t)m * (K / 32) + b] = s[scale_record_offset(m, t / 4, 4 * gq + t % 4, ks4)];
      }
  } else {
    // INT4: FP6 codes back to canonical nibbles
    const uint8_t* tail = q + code_bytes(M, steps);
    std::memset(xq, 0, (size_t)M * (K / 2));
    for (int32_t m = 0; m < M; ++m)
      for (int32_t t = 0; t < steps; ++t)
        for (int sl = 0; sl < 4; ++sl) {
          uint32_t d[6];
          std::memcpy(d, q + i4_main_offset(m, t, sl, steps), 16);
          std::memcpy(d + 4, tail + i4_tail_offset(m, t, sl, steps), 8);
          uint8_t c[32];
          unpack6(d, c);
          for (int j = 0; j < 32; ++j) {
            const int32_t k = t * kStep + 32 * sl + j;
            xq[(size_t)m * (K / 2) + k / 2] |= (uint8_t)((int4_of_e2m3(c[j]) & 0xF) << ((k & 1) * 4));
          }
        }
    const uint8_t* s = base + L.xs_off;
    uint16_t* xs16 = reinterpret_cast<uint16_t*>(xs);
    for (int32_t m = 0; m < M; ++m)
      for (int32_t t = 0; t < steps; ++t)
        for (int G = 0; G < 2; ++G)
          std::memcpy(xs16 + (size_t)m * (K / 64) + 2 * t + G, s + i4_xscale_offset(m, t, G, steps), 2);
  }
  if (z && rank > 0) {
    const int32_t rp = rank_pad(rank);
    const uint16_t* zp = reinterpret_cast<const uint16_t*>(base + L.z_off);
    for (int32_t m = 0; m < M; ++m)
      for (int32_t j = 0; j < rank; ++j) {
        const uint16_t* c = zp + (size_t)m * 2 * rp + 64 * (j / 32) + (j % 32);
        z[(size_t)m * rank + j] = (float)(double_from_bf16(c[0]) + double_from_bf16(c[32]));
      }
  }
  return SVDQ_OK;
}

}  // extern "C"
