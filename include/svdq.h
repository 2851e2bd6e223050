/*
 * svdq.h -- C ABI of the MI355X (gfx950) SVDQuant W4A4 + low-rank linear layer.
 *
 * The layer computes (Zhou, SVDQuant reading notes, sec. 4.2, Eq. (7)):
 *
 *     Y = Q(X diag(lambda)^-1) Q(R) + (X diag(lambda)^-1 L1) L2 + bias
 *
 * with X [M, K] bf16 activations, lambda [K] the smoothing vector (Eq. (3),
 * (4)), L1 [K, r] / L2 [r, N] bf16 low-rank factors (Eq. (10)), R [K, N] the
 * residual quantized to 4 bits and Y [M, N] bf16.  Two 4-bit formats:
 *   SVDQ_INT4_G64   symmetric INT4 codes -7..7, one fp16 scale per 64
 *                   elements along K (notes sec. 2.2 Eq. (1) and sec. 8);
 *   SVDQ_MXFP4_G32  E2M1 codes, one E8M0 power-of-two scale per 32
 *                   elements along K (AutoRound SVDQuant doc, export
 *                   section: MXFP4 E2M1, group 32, symmetric, dynamic
 *                   activation quantization).
 *
 * Conventions for every entry point:
 *  - Plain pointers and sizes only.  "host" pointers are CPU memory,
 *    "device" pointers are HIP device memory on the current device.
 *  - The caller owns every buffer.  The library allocates no device memory
 *    and keeps no global mutable state apart from a write-once per-device
 *    record of the gfx950 check (atomic); all entry points are re-entrant.
 *  - Device calls are asynchronous on `stream` (a hipStream_t, NULL = the
 *    default stream) and never synchronize.  All arguments are validated on
 *    the host before any HIP call; a failed validation returns an error and
 *    launches nothing.
 *  - Errors are returned as svdq_status; nothing aborts or throws across
 *    the ABI.  Host entry points leave their outputs unspecified on error.
 *  - bf16 and fp16 values travel as uint16_t bit patterns.
 *  - Matrices are row-major.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVDQ_ABI_VERSION 8   /* 8: MXFP4 with the OCP shared-exponent rule as a format */
#define SVDQ_MAX_RANK 128   /* msModelSlim doc, svd_res: rank not above 128 recommended */

typedef enum svdq_status {
  SVDQ_OK = 0,
  SVDQ_ERR_ARG = 1,          /* NULL pointer, value out of range */
  SVDQ_ERR_SHAPE = 2,        /* M, K, N or rank not supported */
  SVDQ_ERR_ALIGN = 3,        /* device pointer not 16-byte aligned */
  SVDQ_ERR_UNSUPPORTED = 4,  /* unknown format, or the device is not gfx950 */
  SVDQ_ERR_WORKSPACE = 5,    /* workspace smaller than svdq_workspace_bytes() */
  SVDQ_ERR_NUMERIC = 6,      /* NaN/Inf in prepare inputs, or the eigen solver did not converge */
  SVDQ_ERR_DEVICE = 7        /* a HIP call failed */
} svdq_status;

/* SVDQ_W8A8: 8-bit codes -127..127 with one fp32 scale per row, i.e. per
 * token for activations (dynamic) and per out-feature for weights (Zhou
 * notes sec. 8, the 8-bit setting).
 * SVDQ_MXFP4_G32_OCP: MXFP4 with the OCP Microscaling v1.0 shared-exponent
 * rule, e = floor(log2(amax)) - 2 clamped to [-127, 127], elements rounded
 * to E2M1 and saturated at +-6 (the pages name MXFP4 blocks without a scale
 * rule: msModelSlim doc, "per_block mxfp4 minmax").  SVDQ_MXFP4_G32 takes the
 * smallest e with amax <= 6 * 2^e (no clipping).  Both share every layout. */
typedef enum svdq_format {
  SVDQ_INT4_G64 = 0, SVDQ_MXFP4_G32 = 1, SVDQ_W8A8 = 2, SVDQ_MXFP4_G32_OCP = 3
} svdq_format;

/* ------------------------------------------------------------------------
 * Shape rules (checked by every entry point):
 *   K % 128 == 0, 128 <= K <= 65536; N % 16 == 0, 16 <= N <= 262144;
 *   1 <= M <= 1048576 (no alignment; the tail rows are masked);
 *   M * K <= 2^32 and N * K <= 2^32 for the device path (4-bit code buffers
 *   below 2 GiB);
 *   0 <= rank <= SVDQ_MAX_RANK and rank % 16 == 0 (rank 0 = plain W4A4).
 * ---------------------------------------------------------------------- */

/* ---------------------------- device layer ---------------------------- */

/* One prepared layer in kernel layout.  All pointers are device pointers,
 * 16-byte aligned, caller-owned and never freed by the library.  The buffers
 * are produced on the host by svdq_kernel_layout() and copied to the device
 * unchanged; their sizes come from svdq_layer_sizes(). */
typedef struct svdq_layer {
  int32_t K, N, rank, fmt;       /* rank = total low-rank width (r, or r + LoRA k) */
  const float*    smooth_inv;    /* [K] fp32 1/lambda */
  const uint8_t*  wq;            /* weight codes, kernel layout (wq_bytes) */
  const uint8_t*  ws;            /* weight scales, kernel layout (ws_bytes) */
  const uint16_t* l1k;           /* down factor, kernel layout (l1k_bytes); unused if rank == 0 */
  const uint16_t* l2k;           /* up factor, kernel layout (l2k_bytes); unused if rank == 0 */
  const uint16_t* bias;          /* [N] bf16, or NULL for no bias */
} svdq_layer;

typedef struct svdq_sizes {
  size_t wq_bytes, ws_bytes, l1k_bytes, l2k_bytes;
  size_t wq_canon_bytes, ws_canon_bytes;   /* canonical codes [N, K/2] (4-bit) or [N, K] (8-bit) and
                                              scales [N, K/G] (4-bit) or [N] fp32 (8-bit) */
} svdq_sizes;

/* Byte sizes of the kernel-layout and canonical buffers of a layer.
 * Errors: SVDQ_ERR_ARG (out NULL), SVDQ_ERR_SHAPE, SVDQ_ERR_UNSUPPORTED (fmt).
 *
 * Kernel layouts (K in steps of 128 elements):
 *   MXFP4 codes: 64 bytes per row-step in canonical byte order, in 1 KB
 *           units of 16 rows x one step, ordered [row / 16][step];
 *           16-byte slot 4 (row % 16) + q of a unit holds chunk
 *           q ^ (((r >> 1) & 1) | ((r >> 2) & 2)) of the row-step, r = row;
 *           rows are padded to a multiple of 16
 *   MXFP4 scale records (weights and activations): 16 bytes per row and 4
 *           steps (4 dwords), in 1 KB units of 64 rows ordered
 *           [row / 64][4-step group]; dword d of row r at unit dword
 *           64 (r % 64 / 16) + 16 d + r % 16; weight rows are first permuted
 *           inside each 64-row block, row 32 p + 8 j + 4 h + i (i, j < 4,
 *           h < 2) taking the place of row 16 (2 p + h) + 4 j + i; block
 *           b = 4t + g (32 elements) at record byte 4 g + t % 4
 *   INT4 codes: each code q (-7..7) is the FP6 E2M3 value q (sign bit 5,
 *           exponent bits 3-4 biased by 1, mantissa bits 0-2; exact for
 *           these integers), the operand type of the scaled 32x32x64 MFMA.
 *           A row-step holds 4 slices s = 2 G + h (elements 64 G + 32 h ..
 *           +32), each 32 six-bit codes packed in 6 dwords (element j at
 *           bits 6 j).  Dwords 0-3 of every slice (the main part) are stored
 *           in 1 KB units of 16 rows x one step ordered [row / 16][step],
 *           slot 4 (row % 16) + (s ^ ((row >> 2) & 3)); dwords 4-5 (the
 *           tail) follow all main parts, in 1 KB units of 32 rows x one step
 *           ordered [row / 32][step], at unit byte 256 s + 8 (row % 32)
 *   INT4 scales: 512-byte units of 128 rows x one step ordered
 *           [row / 128][step]; activations: dword row % 128 holds the fp16
 *           scales of the step's groups 2t (low half) and 2t + 1; weights:
 *           fp16 index 128 G + row % 128 holds group 2t + G
 *   W8A8: codes in the MXFP4 code layout with 64 elements per step (byte b
 *           of step t is element 64 t + b, canonical order), so a row has
 *           K/64 steps; weight scales are the canonical fp32 [N]
 * Padding rows, steps and records hold zero codes, scale 127 (MXFP4) or 0 (INT4). */
svdq_status svdq_layer_sizes(int32_t K, int32_t N, int32_t rank, int32_t fmt, svdq_sizes* out);

/* --------------------------- workspace ------------------------------- */

/* Per-call device workspace.  Regions, each 256-byte aligned:
 *   xq   activation codes in the codes layout above (rows padded to 16;
 *        ceil(M/16) * 16 * K/2 bytes, K bytes per row for W8A8; INT4: the
 *        main parts, ceil(M/16) * 16 * K/2 bytes, then the tails,
 *        ceil(M/32) * 32 * K/4 bytes; padding rows are not written)
 *   xs   activation scales: MXFP4 scale records (ceil(M/64) * 64 *
 *        ceil(K/512) * 16 bytes); INT4 scale units (ceil(M/128) * K/128 *
 *        512 bytes); W8A8 fp32 [M] per token scales (ceil(M/16) * 64 bytes)
 *   z    down projection Z: per row and 32-column chunk of the rank
 *        (rounded up to 32), 32 bf16 values hi then 32 bf16 values lo with
 *        hi + lo = Z to about 2^-17 relative (M * rank_pad * 4 bytes)
 * svdq_unpack_activations() turns a host copy into canonical form. */
typedef struct svdq_ws_layout {
  size_t xq_off, xq_bytes, xs_off, xs_bytes, z_off, z_bytes, total;
  int32_t zsplit;                 /* number of K splits of the down projection */
} svdq_ws_layout;

svdq_status svdq_workspace_layout(int32_t M, int32_t K, int32_t rank, int32_t fmt, svdq_ws_layout* out);
size_t svdq_workspace_bytes(int32_t M, int32_t K, int32_t rank, int32_t fmt);  /* 0 on invalid shape */

/* ------------------------- host preparation --------------------------- */

/* Running per-channel absolute maximum over calibration activations
 * (notes, Algorithm 1 step 1: statistics from calibration inputs):
 * amax[k] = max(amax[k], |x[i,k]|) for all rows i.  x: host [rows, K] bf16;
 * amax: host [K] fp32, in/out (start from zeros).  Errors: ARG, NUMERIC
 * (NaN/Inf in x). */
svdq_status svdq_calib_absmax(const uint16_t* x, int64_t rows, int32_t K, float* amax);

typedef struct svdq_prepare_opts {
  int32_t        lora_rank;       /* k >= 0, rank + k <= SVDQ_MAX_RANK, multiple of 16 */
  const float*   lora_a;          /* host [K, k] (adapter A, unsmoothed coordinates) */
  const float*   lora_b;          /* host [k, N] */
  float          lora_strength;   /* absorbed into B */
  int32_t        threads;         /* host threads; 0 = OMP_NUM_THREADS if set, else the CPUs the
                                     process may run on (at most 64) */
  int32_t        max_iters;       /* eigen solver iteration cap per value; 0 = default, < 0 forces
                                     SVDQ_ERR_NUMERIC (test hook) */
  int32_t        residual_iters;  /* 0 or 1: one SVD; T > 1: residual iteration (below); <= SVDQ_MAX_RESIDUAL_ITERS */
  int32_t        residual_early_stop; /* nonzero: stop at the first iteration worse than the best */
  int32_t        has_beta;        /* nonzero: lambda uses the weight exponent `beta` below */
  double         beta;            /* in [0, 1]; when has_beta == 0 the exponent is 1 - alpha */
} svdq_prepare_opts;

#define SVDQ_MAX_RESIDUAL_ITERS 64

/* Canonical host outputs of svdq_prepare (caller-allocated). */
typedef struct svdq_prepared {
  float*    lambda;       /* [K] fp32 lambda (optional, may be NULL) */
  float*    smooth_inv;   /* [K] fp32 1/lambda (required) */
  uint16_t* l1;           /* [K, rank + k] bf16 L1' = [L1 | bf16(D A)] (required if rank + k > 0) */
  uint16_t* l2;           /* [rank + k, N] bf16 L2' = [L2 ; bf16(s B)] (required if rank + k > 0) */
  float*    residual;     /* [K, N] fp32 R (optional) */
  double*   sigma;        /* [rank] leading singular values of diag(lambda) W (optional) */
  uint8_t*  wq;           /* [N, K/2] canonical codes of R^T (required) */
  uint8_t*  ws;           /* [N, K/G] canonical scales: fp16 bits (INT4) or E8M0 bytes (MXFP4) (required) */
  double*   iter_errors;  /* [max(1, residual_iters)] ||W~ - L1b L2b - Q(R)||_F of every iteration run,
                             NaN for those not run (optional) */
  int32_t*  best_iter;    /* index of the kept iteration (optional) */
} svdq_prepared;

/* Offline preparation of one layer (notes, Algorithm 1; AutoRound doc,
 * "Residual iteration" and "Smooth search"):
 *   lambda_i = amaxX_i^alpha / amaxW_i^beta        (Eq. (4), beta = 1 - alpha unless
 *                                                   opts->has_beta; 1 when either is 0)
 *   W~ = diag(lambda) W                            (Eq. (3))
 *   L1 = U_r S_r, L2 = V_r^T of W~                 (Eq. (10), exact top-r)
 *   L1b, L2b = bf16(L1), bf16(L2); R = W~ - L1b L2b (fp64, stored fp32)
 *   codes/scales = RTN of R^T grouped along K in `fmt`.
 * With residual_iters = T > 1, iteration t >= 2 takes the top-r split of
 * W~ - Q(R_{t-1}) instead of W~ (Q = the RTN quantize-dequantize above) and
 * forms R_t = W~ - L1b L2b again.  Every iteration is scored by the weight
 * reconstruction error ||W~ - L1b L2b - Q(R_t)||_F and the best one is
 * returned; with residual_early_stop the loop ends at the first iteration
 * that scores worse than the best so far.
 * W: host [K, N] fp32; act_amax: host [K] fp32 (svdq_calib_absmax);
 * alpha in [0, 1].  A grouped projection (e.g. Q|K|V) is passed as the
 * column concatenation of its weights: one lambda, one shared L1, and the
 * separate up factors are the column blocks of L2.
 * Errors: ARG, SHAPE, UNSUPPORTED, NUMERIC (NaN/Inf inputs, solver failure). */
svdq_status svdq_prepare(const float* W, const float* act_amax, int32_t K, int32_t N, double alpha,
                         int32_t rank, int32_t fmt, const svdq_prepare_opts* opts, svdq_prepared* out);

/* ---------------------------- smooth search --------------------------- */

/* Candidate exponent pairs of the smooth search (AutoRound doc, "Smooth
 * search"): (0, 0), then (a/G, 0) for a = 1 .. G-1, then (a/G, 1 - a/G) for
 * the same a, in that order.  Returns the count 2G - 1 (39 for G = 20), or 0
 * if G is outside [2, 1000]; fills alpha[] and beta[] (host) when both are
 * non-NULL. */
int32_t svdq_smooth_candidates(int32_t grids, double* alpha, double* beta);

typedef struct svdq_search_opts {
  int32_t grids;                  /* G; 0 = 20 */
  int32_t residual_iters;         /* per candidate, as in svdq_prepare_opts */
  int32_t residual_early_stop;
  int32_t threads;                /* host threads of each preparation; 0 as in svdq_prepare_opts */
} svdq_search_opts;

typedef struct svdq_search_result {
  int32_t count;                  /* number of candidates scored (2G - 1) */
  int32_t best;                   /* index of the winner in candidate order, -1 if none is finite */
  double  alpha, beta;            /* the winner's exponents */
  double* errors;                 /* host [count] scores, NaN where a candidate could not be
                                     prepared (optional, caller-allocated) */
  int32_t best_iter;              /* the winner's kept residual iteration (0 without residual
                                     iteration), -1 if none is finite */
} svdq_search_result;

/* Reservoir selection of calibration calls (AutoRound doc, "Smooth search":
 * each group keeps at most k calls, chosen by reservoir sampling).  Algorithm
 * R (Vitter 1985): calls 0..k-1 fill the reservoir; call i >= k draws
 * j = hi64(r * (i + 1)) with r the next SplitMix64 output (Steele, Lea and
 * Flood 2014; state starts at `seed`) and replaces slot j when j < k.
 * Writes the min(n_calls, k) kept indices in increasing order to out (host,
 * caller-allocated) and returns their count; 0 if n_calls <= 0 or k <= 0;
 * -1 if out is NULL. */
int64_t svdq_reservoir_select(int64_t n_calls, int64_t k, uint64_t seed, int64_t* out);

/* Device workspace bytes of svdq_smooth_search (0 on an invalid shape). */
size_t svdq_search_workspace_bytes(int32_t M, int32_t K, int32_t N, int32_t rank, int32_t fmt);

/* Smooth-factor grid search of one layer (AutoRound doc, "Smooth search").
 * lambda_i = x_span_i^alpha / w_span_i^beta with x_span the per-channel
 * absolute maximum of the calibration rows x_cal and w_span that of the
 * weight rows.  Every candidate is prepared as svdq_prepare does, run
 * through svdq_linear_forward on x_cal (no bias) and scored by
 * ||Y - x_cal W||_F / ||x_cal W||_F, with the reference x_cal W computed on
 * the device in fp32.  With opts' residual iteration, every iteration of a
 * candidate is scored by that output error (AutoRound doc, "Residual
 * iteration": calibration output error when smooth is on, in place of the
 * weight error svdq_prepare uses), the best iteration is kept (early stop
 * at the first score above the best) and its score is the candidate's.
 * The finite smallest score wins (the earlier candidate on ties).
 * W: host [K, N] fp32.  x_cal: device [M, K] bf16, 16-byte aligned.
 * ws: device workspace of svdq_search_workspace_bytes(), 256-byte aligned.
 * best (optional): receives the winner's lambda, smooth_inv, l1, l2, wq and
 * ws as svdq_prepare would write them (other fields are ignored).
 * Blocks the calling thread: it synchronizes `stream` once per candidate.
 * Errors: ARG, SHAPE, ALIGN, WORKSPACE, UNSUPPORTED, NUMERIC (non-finite W
 * or x_cal, an all-zero reference, or no finite score), DEVICE. */
svdq_status svdq_smooth_search(const float* W, int32_t K, int32_t N, int32_t rank, int32_t fmt,
                               const uint16_t* x_cal, int32_t M, const svdq_search_opts* opts, void* ws,
                               size_t ws_bytes, void* stream, svdq_search_result* res, svdq_prepared* best);

/* RTN quantization of a host [rows, K] fp32 matrix, grouped along K, into
 * canonical codes [rows, K/2] (element 2j in the low nibble of byte j) and
 * canonical scales [rows, K/G] (fp16 bits or E8M0 bytes); for W8A8 one
 * group per row: codes [rows, K] int8 and scales [rows] fp32 (Zhou notes
 * sec. 8).  Errors: ARG, SHAPE. */
svdq_status svdq_pack_host(const float* x, int32_t rows, int32_t K, int32_t fmt,
                           uint8_t* codes, uint8_t* scales);

/* LoRA attach (notes sec. 7, Eq. (13)): l1_out = [l1 | bf16(diag(lambda) A)],
 * l2_out = [l2 ; bf16(strength B)].  The residual codes are unchanged.
 * l1: [K, rank] bf16, l2: [rank, N] bf16, A: [K, k] fp32, B: [k, N] fp32;
 * l1_out: [K, rank + k], l2_out: [rank + k, N].  Errors: ARG, SHAPE. */
svdq_status svdq_attach_lora(const float* lambda, const uint16_t* l1, const uint16_t* l2,
                             int32_t K, int32_t N, int32_t rank, const float* A, const float* B,
                             int32_t k, float strength, uint16_t* l1_out, uint16_t* l2_out);

/* Canonical host buffers -> kernel-layout host buffers (sizes from
 * svdq_layer_sizes).  l1 may be NULL when rank == 0.  The down factor L1'
 * (bf16) is stored in the order of the quantize kernel's MFMA operand,
 * [step][s 0..3][16-column tile 0..rank/16-1][lane 0..63][i 0..7] holding
 * L1'[128 step + 32 (lane / 16) + 8 s + i][16 tile + lane % 16];
 * the up factor as L2'^T [N][rank rounded up to 32] (0 past rank). */
svdq_status svdq_kernel_layout(int32_t K, int32_t N, int32_t rank, int32_t fmt,
                               const float* smooth_inv, const uint8_t* wq, const uint8_t* ws,
                               const uint16_t* l1, const uint16_t* l2,
                               uint8_t* wq_k, uint8_t* ws_k, uint16_t* l1k, uint16_t* l2k);

/* Host copy of a workspace -> canonical activation codes [M, K/2] ([M, K]
 * for W8A8), scales [M, K/G] ([M] fp32 for W8A8) and (if z != NULL) the
 * summed down projection z [M, rank] fp32. */
svdq_status svdq_unpack_activations(const void* ws_host, int32_t M, int32_t K, int32_t rank, int32_t fmt,
                                    uint8_t* xq, uint8_t* xs, float* z);

/* ---------------------------- device path ----------------------------- */

/* K-A: fused smoothing + group absmax + 4-bit quantize/pack + lora_down
 * (notes, Algorithm 2 steps 1-3; AutoRound/msModelSlim "lora_down").
 * Reads X once: x~ = fp32(x * smooth_inv), per-group scales and codes into
 * the workspace, z = x~ L1' as bf16 hi + lo pairs.  W8A8: the per-token
 * scale needs the whole row's maximum, so the codes are written in a second
 * pass over the block's rows of X (a cache re-read).
 * X: device [M, K] bf16.  Errors: ARG, SHAPE, ALIGN, WORKSPACE, UNSUPPORTED, DEVICE. */
svdq_status svdq_quantize_lora_down(const svdq_layer* layer, const uint16_t* X, int32_t M,
                                    void* ws, size_t ws_bytes, void* stream);

/* K-B: W4A4 GEMM with per-group scales, lora_up epilogue (z L2') and bias,
 * one bf16 store of Y (notes, Algorithm 2 steps 4-7).  W8A8: int8 GEMM with
 * exact int32 accumulation, scaled by s_x[m] s_w[n] after the K loop.
 * Y: device [M, N] bf16.  Errors: as above. */
svdq_status svdq_gemm_lora_up(const svdq_layer* layer, const void* ws, size_t ws_bytes, int32_t M,
                              uint16_t* Y, void* stream);

/* K-A then K-B on `stream`. */
svdq_status svdq_linear_forward(const svdq_layer* layer, const uint16_t* X, int32_t M, uint16_t* Y,
                                void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as svdq_linear_forward without a workspace argument.  The
 * workspace is a file-scope device array of SVDQ_NOALLOC_MAX_WORKSPACE bytes
 * in the library, one per GPU, held until the process ends; its device
 * address is looked up on the first call on each device.  The call
 * allocates nothing.  Layers whose svdq_workspace_bytes(M, K, rank, fmt)
 * exceeds the maximum return SVDQ_ERR_WORKSPACE.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams or threads) race and must be serialized by the caller.
 * Errors: ARG, SHAPE, ALIGN, WORKSPACE, UNSUPPORTED, DEVICE. */
#define SVDQ_NOALLOC_MAX_WORKSPACE (32u << 20)
svdq_status svdq_linear_forward_noalloc(const svdq_layer* layer, const uint16_t* X, int32_t M, uint16_t* Y,
                                        void* stream);

/* The same layer computed by four separate kernels, the arrangement whose
 * cost the notes weigh against the fused kernels (Zhou notes, sec. 6.1: run
 * unfused, the low-rank branch adds a large share of the 4-bit layer's time,
 * mostly memory traffic): quantize only; the down projection as a second
 * pass over X; the W4A4 GEMM with bias storing Y; then Y += Z L2' as a
 * read-modify-write of Y.  Same layer, workspace, arguments and errors as
 * svdq_linear_forward; Y is rounded to bf16 twice (after the GEMM and after
 * the add), so it matches the fused result to bf16 rounding, not bitwise. */
svdq_status svdq_linear_forward_unfused(const svdq_layer* layer, const uint16_t* X, int32_t M, uint16_t* Y,
                                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------ misc ---------------------------------- */

const char* svdq_status_str(svdq_status s);
int32_t svdq_abi_version(void);
/* SVDQ_OK if `device` is a gfx950 GPU, SVDQ_ERR_UNSUPPORTED otherwise,
 * SVDQ_ERR_DEVICE if HIP cannot be queried (e.g. no GPU present). */
svdq_status svdq_device_check(int32_t device);

/* Sustained matrix-unit rate of the current device, a diagnostic for pricing
 * the GEMM kernels against what the chip delivers beside its datasheet peak
 * (not part of the layer).  `blocks` blocks of 512 threads (two waves per
 * SIMD; one block per compute unit covers the chip) each issue MFMAs back to
 * back for `iters` iterations with independent accumulators, on operands
 * that change every MFMA (bytes from a fixed integer hash, or all zero when
 * zero_operands != 0) and with no memory traffic in the loop:
 *   kind 0: scaled 16x16x128 FP4 (E2M1, unit scales), 32 per wave and iteration;
 *   kind 1: 32x32x32 int8, 16 per wave and iteration.
 * Each MFMA is 65536 operations, so one launch does blocks * 8 * 32 * iters
 * (kind 0) or blocks * 8 * 16 * iters (kind 1) of them; the caller times the
 * launch on `stream`.  sink: device, blocks * 512 floats, written so the
 * work is kept.  marks: device, blocks * 16 uint64 (per wave: shader-clock
 * cycles, then 100 MHz wall-clock ticks, of its loop), or NULL.
 * Errors: ARG (kind not 0/1, blocks outside 1..65535, iters outside
 * 1..2^20, NULL sink), ALIGN (sink not 4-byte or marks not 8-byte aligned),
 * UNSUPPORTED (not gfx950), DEVICE. */
svdq_status svdq_mfma_rate_probe(int32_t kind, int32_t zero_operands, int32_t blocks, int32_t iters,
                                 float* sink, uint64_t* marks, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SVDQ_H */
