/*
 * metis_fp4.h -- C ABI of libmetis_fp4.so: the spectral-domain FP4 linear
 * layer (randomized split + block FP4 quantization + W4A4G4 GEMMs) for
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "Metis: Training LLMs with FP4 Quantization" (arXiv 2509.00404),
 * abstract; SII open-source-week post on Metis, §2.3-§2.4. A matrix is split
 * into a dominant low-rank part U_k diag(S_k) V_k^T, found by a random
 * projection or by sparse column sampling, and a long-tail residual R; each
 * part is quantized to FP4 separately and the linear layer's three GEMMs run
 * on the quantized parts.
 *
 * Conventions for every call
 *  - Array pointers are DEVICE pointers owned by the caller. The library never
 *    allocates or frees memory, never synchronizes the device and keeps no
 *    global state: calls are re-entrant and may run on any stream. (The one
 *    exception, spectral_fp4_linear_fwd_noalloc, uses a static per-GPU
 *    scratch array instead of a workspace argument.)
 *  - All work is enqueued on `stream` (asynchronous). Outputs are valid once
 *    the stream reaches that point.
 *  - Arguments are validated on the host before any HIP call; a failed check
 *    returns METIS_ERR_INVALID / METIS_ERR_UNSUPPORTED / METIS_ERR_WORKSPACE
 *    and enqueues nothing. A failed launch returns METIS_ERR_HIP.
 *  - Matrices are row-major with an explicit leading dimension (elements).
 *  - FP4 blocks always run along the last (contiguous) axis of the stored
 *    matrix; for a GEMM operand that is the contraction axis.
 *  - Inputs containing NaN or Inf give undefined (but memory-safe) results.
 *  - Empty matrices (a zero dimension) are valid and enqueue nothing.
 */
#ifndef METIS_FP4_H
#define METIS_FP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  METIS_OK = 0,
  METIS_ERR_INVALID = 1,     /* bad pointer, shape, leading dimension or missing operand */
  METIS_ERR_UNSUPPORTED = 2, /* a valid request this build does not implement */
  METIS_ERR_WORKSPACE = 3,   /* ws == NULL or ws_bytes below the matching *_workspace_bytes() */
  METIS_ERR_HIP = 4,         /* a HIP launch failed */
  METIS_ERR_TOO_LARGE = 5    /* the request needs more than a fixed-size static scratch */
} metis_status_t;

/* FP4 block formats (the pages name MXFP4 and NVFP4: SII post, project
 * highlights and §2.2). Bit layouts: OCP Microscaling Formats v1.0 (E2M1
 * elements, E8M0 scale per 32) and NVIDIA's NVFP4 (E2M1, E4M3 scale per 16,
 * one fp32 scale per tensor). */
typedef enum { METIS_MXFP4 = 0, METIS_NVFP4 = 1 } metis_fmt_t;

/* Storage type of a dense input. */
typedef enum { METIS_F32 = 0, METIS_BF16 = 1 } metis_dtype_t;

/* How the dominant subspace is sketched ("Metis" abstract: preservation via
 * random projection, and via sparse random sampling). */
typedef enum {
  METIS_OMEGA_GAUSSIAN = 0, /* omega: n x l bf16 row-major Gaussian test matrix */
  METIS_OMEGA_COLUMNS = 1   /* omega: int32 J[l], distinct column ids in [0, n) */
} metis_omega_t;

/* One FP4 matrix (rows x cols), blocks along cols.
 *  codes:        rows * cols / 2 bytes, row-major; element 2j of a row sits in
 *                the low nibble of byte j, element 2j+1 in the high nibble.
 *                Nibble = E2M1 code: bit 3 sign, bits 2-1 exponent, bit 0 mantissa.
 *  scales:       rows * (cols / B) bytes row-major, B = 32 (MXFP4, E8M0 byte e
 *                means 2^(e-127)) or 16 (NVFP4, E4M3 byte).
 *  tensor_scale: NVFP4 only: one fp32 on the device; NULL for MXFP4.
 * Element value: e2m1(code) * scale (* tensor_scale for NVFP4). */
typedef struct {
  int32_t fmt; /* metis_fmt_t */
  int32_t reserved;
  int64_t rows, cols;
  uint8_t *codes;
  uint8_t *scales;
  float *tensor_scale;
} metis_fp4_t;

/* Quantized split of one m x n tensor A = U diag(S) V^T + R.
 * k == 0 marks an operand that is not split: R_q / Rt_q then hold the
 * quantized tensor itself and U, S, V, Ut_q, Vt_q are unused.
 *  U (m x k), S (k, descending), V (n x k): fp32 row-major factors. Each column
 *      of U has its largest-magnitude entry positive (lowest row on ties).
 *  Ut_q: U^T (k x m) blocked along m;  Vt_q: V^T (k x n) blocked along n.
 *      (Each singular vector is quantized along its length; S stays fp32.)
 *  R_q:  R (m x n) blocked along n -- the operand of a GEMM contracting over n.
 *  Rt_q: R^T (n x m) blocked along m -- the operand of a GEMM contracting over m.
 *      Either residual orientation may be absent (codes == NULL). */
typedef struct {
  int64_t m, n;
  int32_t k;
  int32_t reserved;
  float *U;
  float *S;
  float *V;
  metis_fp4_t Ut_q;
  metis_fp4_t Vt_q;
  metis_fp4_t R_q;
  metis_fp4_t Rt_q;
} metis_split_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *metis_status_str(metis_status_t status);

/* ABI revision of this header (bumped on any incompatible change). */
int32_t metis_abi_version(void);

/* ------------------------------------------------------------------------
 * Block FP4 quantization of a dense matrix (OCP MX v1.0 §6.3 scale rule for
 * MXFP4: shared exponent floor(log2 amax) - 2, clamped to [-127, 127];
 * NVFP4: s_t = max(amax_tensor / 2688, 2^-126), block scale
 * e4m3(amax_block / (6 s_t)), element x / (e4m3 * s_t), each step a correctly
 * rounded fp32 operation). Elements round to nearest E2M1 value, ties to the
 * even code, saturating at +-6; an all-zero block gets scale 0 and +-0 codes.
 *
 *  x:         rows x cols, leading dimension ldx >= cols, type dt.
 *  transpose: 0 -> out is rows x cols blocked along cols;
 *             1 -> out is x^T (cols x rows) blocked along rows.
 *  out:       caller sets fmt, codes, scales (and tensor_scale for NVFP4);
 *             the library writes out->rows and out->cols.
 *  ws:        scratch of fp4_block_quant_workspace_bytes() bytes (0 for MXFP4:
 *             ws may then be NULL).
 * The blocked axis must be a multiple of the block size (32 or 16). */
size_t fp4_block_quant_workspace_bytes(int64_t rows, int64_t cols, metis_fmt_t fmt);
metis_status_t fp4_block_quant(const void *x, metis_dtype_t dt, int64_t rows, int64_t cols, int64_t ldx,
                               int32_t transpose, metis_fp4_t *out, void *ws, size_t ws_bytes,
                               hipStream_t stream);

/* Exact dequantization to fp32: y (in->rows x in->cols, leading dimension
 * ldy >= in->cols) = e2m1(code) * scale (* tensor_scale). */
metis_status_t fp4_block_dequant(const metis_fp4_t *in, float *y, int64_t ldy, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Randomized spectral split (SII post on Metis §2.4 item 1: dominant part and
 * long-tail residual, quantized separately, decomposition done in a
 * low-dimensional space; steps as in Halko-Martinsson-Tropp 2011, Alg. 4.1
 * without power iterations and Alg. 5.1):
 *   Y = A Omega (or A[:, J]);  Q = orth(Y);  B = Q^T A;  B = Ub diag(sigma) W^T;
 *   U = Q Ub[:, :k], S = sigma[:k], V = W[:, :k], column signs fixed as above;
 *   R = A - U diag(S) V^T, quantized in the orientations whose codes != NULL;
 *   U^T and V^T quantized along their length.
 *
 *  A:     m x n (lda >= n) of type dt.
 *  omega: METIS_OMEGA_GAUSSIAN: n x l bf16 row-major (the bits of bfloat16
 *         values); METIS_OMEGA_COLUMNS: int32[l] distinct ids in [0, n)
 *         (ids out of range give undefined values, never an out-of-bounds read).
 *  1 <= k <= l <= min(m, n); k <= 96 and l <= 512 (beyond: METIS_ERR_UNSUPPORTED).
 *  Sketches with l <= 96 keep the l x l problems in LDS; wider ones keep
 *  them in global memory (their Cholesky and tridiagonal reduction take one
 *  launch per 16 pivots or per reflector, so they are launch-bound). m and n
 *  multiples of 32; A
 *  16-byte aligned and lda * sizeof(element) a multiple of 16.
 *  out:   caller provides U, S, V (fp32) and the codes/scales (/tensor_scale)
 *         buffers of Ut_q, Vt_q, R_q and/or Rt_q (each fp4 member's fmt must
 *         equal `fmt`); the library writes m, n, k and the rows/cols fields.
 *  info:  optional device int32 (may be NULL), written with 0 on success or
 *         i > 0 when the sketch is rank deficient (the i-th pivot of its
 *         Cholesky factor broke down); the columns of U from that rank on
 *         then carry S = 0. Read it after synchronizing the stream.
 *  ws:    scratch of metis_split_workspace_bytes() bytes, 256-byte aligned.
 * Results are bitwise reproducible run to run (no atomics in reductions). */
size_t metis_split_workspace_bytes(int64_t m, int64_t n, int32_t l, int32_t k, metis_omega_t kind,
                                   metis_fmt_t fmt);
metis_status_t metis_split(const void *A, metis_dtype_t dt, int64_t m, int64_t n, int64_t lda,
                           const void *omega, metis_omega_t kind, int32_t l, int32_t k, metis_fmt_t fmt,
                           metis_split_t *out, int32_t *info, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* The same split with q power (subspace) iterations after the sketch
 * (Halko-Martinsson-Tropp 2011, Alg. 4.4): with Q = orth(Y), each iteration
 * forms Z = orth(A^T Q) and Y = A Z, Q = orth(Y), every orthonormalization a
 * CholeskyQR2 in fp64 and Z applied as bf16 hi + lo (fp32-accurate). Each
 * iteration adds two passes over A. metis_split is q = 0.
 *  q: 0 <= q <= 16 (beyond: METIS_ERR_UNSUPPORTED); q > 0 needs l <= 96
 *     (beyond: METIS_ERR_UNSUPPORTED); q < 0: METIS_ERR_INVALID.
 *  info: the rank status of the last sketch's Cholesky factor.
 *  ws: metis_split_power_workspace_bytes() bytes (it grows with q > 0).
 * Everything else as for metis_split. */
size_t metis_split_power_workspace_bytes(int64_t m, int64_t n, int32_t l, int32_t k, metis_omega_t kind,
                                         int32_t q, metis_fmt_t fmt);
metis_status_t metis_split_power(const void *A, metis_dtype_t dt, int64_t m, int64_t n, int64_t lda,
                                 const void *omega, metis_omega_t kind, int32_t l, int32_t k, int32_t q,
                                 metis_fmt_t fmt, metis_split_t *out, int32_t *info, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * Mean-residual split (Averis, "Averaging-Induced Residual Splitting", as
 * retold on the zhu318.com page, method paragraphs): the mean over all rows,
 * mu (one value per column), and the residual A - mu broadcast over the rows
 * are quantized separately. The result is the rank-1 split record
 *   U = 1 (m x 1), S = {1}, V = mu (n x 1),  R = A - 1 mu^T,
 * so it enters spectral_fp4_linear_fwd/_bwd and metis_gemm_nt_* like any
 * split operand (the all-ones U is exact in both FP4 formats).
 *  A, dt, m, n, lda, fmt, out, ws, stream: as for metis_split, with k = 1
 *  (out->U holds m floats, S one, V n). mu is summed in fp64 over rows in a
 *  fixed order and rounded once to fp32; R = A - mu is one fp32 subtraction
 *  per element. ws: metis_mean_split_workspace_bytes() bytes, 256-byte
 *  aligned. Errors as for metis_split; bitwise reproducible. */
size_t metis_mean_split_workspace_bytes(int64_t m, int64_t n, metis_fmt_t fmt);
metis_status_t metis_mean_split(const void *A, metis_dtype_t dt, int64_t m, int64_t n, int64_t lda,
                                metis_fmt_t fmt, metis_split_t *out, void *ws, size_t ws_bytes,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * W4A4G4 linear layer ("Metis" abstract: FP4 weights, activations and
 * gradients). Each GEMM is C = A_hat B_hat^T with, for a split operand,
 * A_hat = R_hat + U_hat diag(S) V_hat^T in the orientation it is used in
 * (R_q for contraction over n, Rt_q for contraction over m). The product runs
 * as the FP4 GEMM of the residuals plus a low-rank correction; outputs are
 * fp32. Shapes: X is M x K (tokens x in), W is N x K (out x in), dY is M x N.
 *   fwd:  Y  = X W^T    (M x N)   needs X.R_q,  W.R_q
 *   bwd:  dX = dY W     (M x K)   needs dY.R_q, W.Rt_q
 *         dW = dY^T X   (N x K)   needs dY.Rt_q, X.Rt_q
 * All operands must share one format. ws: metis_linear_workspace_bytes()
 * bytes (256-byte aligned); dY may be NULL in the query for fwd only. */
size_t metis_linear_workspace_bytes(const metis_split_t *X, const metis_split_t *W, const metis_split_t *dY);
metis_status_t spectral_fp4_linear_fwd(const metis_split_t *X, const metis_split_t *W, float *Y, int64_t ldy,
                                       void *ws, size_t ws_bytes, hipStream_t stream);
/* The forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * spectral_fp4_linear_fwd with its workspace taken from a static device array
 * of METIS_NOALLOC_SCRATCH_BYTES in the library instead of a ws argument. The
 * call itself allocates nothing; each GPU the library runs on holds its own
 * copy of the array from the library's load until the process ends. Inputs
 * and Y are the caller's, as for spectral_fp4_linear_fwd, and the result is
 * the same bit for bit.
 *  - Work is enqueued on `stream`, which must belong to the current device.
 *  - A forward whose metis_linear_workspace_bytes(X, W, NULL) exceeds
 *    METIS_NOALLOC_SCRATCH_BYTES returns METIS_ERR_TOO_LARGE and enqueues
 *    nothing (64 MiB covers 8192 tokens x 4096 x 14336 at k = 64).
 *  - Every call on one GPU shares that GPU's array, and the array keeps the
 *    last call's contents (nothing in it needs to start at zero). Calls that
 *    overlap on one GPU (concurrent streams, or host threads without
 *    ordering) race on it: serialize them.
 * Other errors as for spectral_fp4_linear_fwd; METIS_ERR_HIP also when the
 * array's device address cannot be looked up. */
#define METIS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
metis_status_t spectral_fp4_linear_fwd_noalloc(const metis_split_t *X, const metis_split_t *W, float *Y,
                                               int64_t ldy, hipStream_t stream);

/* dX or dW may be NULL to skip that product. */
metis_status_t spectral_fp4_linear_bwd(const metis_split_t *dY, const metis_split_t *X, const metis_split_t *W,
                                       float *dX, int64_t lddx, float *dW, int64_t lddw, void *ws,
                                       size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The two halves of one GEMM C = A_hat B_hat^T (rows of C from operand a,
 * columns from operand b; a_trans / b_trans select the orientation each
 * operand is used in: 0 -> R_q, contraction over its n; 1 -> Rt_q,
 * contraction over its m). spectral_fp4_linear_fwd/bwd are prepare + main.
 *  prepare: the skinny FP4 products R_a F_b, R_b F_a, F_a^T F_b and the bf16
 *           correction panels, written into ws;
 *  main:    the FP4 GEMM of the residuals plus the low-rank correction read
 *           from ws (left there by prepare on the same stream), fp32 output.
 * Splitting them lets a caller run the next prepare (in another workspace)
 * while a main runs, or time the main kernel alone. ws holds
 * metis_gemm_nt_workspace_bytes() bytes, 256-byte aligned. */
size_t metis_gemm_nt_workspace_bytes(const metis_split_t *a, int32_t a_trans, const metis_split_t *b,
                                     int32_t b_trans);
metis_status_t metis_gemm_nt_prepare(const metis_split_t *a, int32_t a_trans, const metis_split_t *b,
                                     int32_t b_trans, void *ws, size_t ws_bytes, hipStream_t stream);
metis_status_t metis_gemm_nt_main(const metis_split_t *a, int32_t a_trans, const metis_split_t *b, int32_t b_trans,
                                  float *C, int64_t ldc, const void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Adaptive spectral learning rate (SII post on Metis, §2.4 item 2; the
 * earlier version's abstract, chatpaper.ai page, item (ii)): the gradient
 * along a split's mid and low singular directions is scaled up by the
 * inverse of its normalized singular value, the dominant directions and the
 * unresolved tail R left as they are. With the split G = U diag(S) V^T + R of
 * the gradient (metis_split of G):
 *   gamma_i = min(gamma_max, max(1, S[r_ref] / S_i))  (1 where S_i = 0),
 *   G <- G + U diag(S (gamma - 1)) V^T,   in place.
 *  G:  m x n fp32, leading dimension ldg >= n (device).
 *  U (m x k), S (k, descending), V (n x k): fp32 row-major, as in a split
 *      record of G (device).
 *  1 <= k <= 96, 0 <= r_ref < k, gamma_max >= 1 (else METIS_ERR_INVALID;
 *  k > 96: METIS_ERR_UNSUPPORTED).
 * The rank-k term is summed in fp32 in ascending i and added to G once. */
metis_status_t metis_spectral_lr_rescale(float *G, int64_t m, int64_t n, int64_t ldg, const float *U,
                                         const float *S, const float *V, int32_t k, int32_t r_ref, float gamma_max,
                                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * Dual-range regularizer (SII post on Metis, §2.4 item 3; chatpaper.ai
 * abstract, item (iii)): a penalty that restrains oversized values and
 * suppresses near-zero ones, compressing a parameter tensor's range. Two-sided
 * hinge on each element w of W:
 *   loss = lam_hi sum relu(|w| - tau_hi)^2 + lam_lo sum_{w != 0} relu(tau_lo - |w|)^2,
 *   dloss/dw = 2 lam_hi relu(|w| - tau_hi) sign(w) - 2 lam_lo relu(tau_lo - |w|) sign(w).
 *  W:     rows x cols of type dt (leading dimension ldw >= cols; cols % 8 == 0;
 *         16-byte aligned rows).
 *  grad:  optional fp32 rows x cols (ldg >= cols, 16-byte aligned rows): the
 *         gradient, stored (accumulate == 0) or added to what is there
 *         (accumulate != 0). Each gradient value is formed in fp64 and rounded
 *         once to fp32 (after the addition when accumulating).
 *  loss:  optional device fp64 scalar; needs ws of
 *         metis_dual_range_workspace_bytes() bytes (8-byte aligned), and is
 *         summed in a fixed order (bitwise reproducible).
 *  0 <= tau_lo <= tau_hi, lam_lo, lam_hi >= 0 (else METIS_ERR_INVALID). */
size_t metis_dual_range_workspace_bytes(void);
metis_status_t metis_dual_range_reg(const void *W, metis_dtype_t dt, int64_t rows, int64_t cols, int64_t ldw,
                                    float tau_lo, float tau_hi, float lam_lo, float lam_hi, float *grad, int64_t ldg,
                                    int32_t accumulate, double *loss, void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* METIS_FP4_H */
