/*
 * bfly.h -- C ABI of libbfly: the learnable butterfly rotation and its fused
 * round-to-nearest quantization, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are the pages' titles and sections):
 *
 *   Q(theta) is the product of L = log2(n) Givens stages, Q = B_{L-1} ... B_0.
 *   Stage s rotates, for every i whose bit s is clear, the pair (i, j = i + 2^s)
 *   by its own angle t = theta[s][p], where p = (i >> (s+1)) * 2^s + (i mod 2^s)
 *   ranks the pair among the stage's pairs by increasing i:
 *       (u_i, u_j) <- (cos t * u_i - sin t * u_j,  sin t * u_i + cos t * u_j).
 *   That is n log2(n) / 2 angles and O(n log n) work per row, orthogonal for
 *   every theta ("ButterflyQuant: Ultra-low-bit LLM Quantization through
 *   Learnable Orthogonal Butterfly Transforms", abstract).  With every angle
 *   pi/4, Q times diag((-1)^popcount(i)) is the Sylvester Hadamard matrix
 *   (duidaima.com write-up of ButterflyQuant, section "butterfly").
 *
 *   Rows are rotated independently.  Applied to activation rows this gives
 *   Q x; applied to the rows of a weight matrix W it gives the rows of W Q^T,
 *   so that W x = (W Q^T)(Q x) (ButterflyQuant abstract, computational
 *   invariance).  The stage order (s = 0 first), the pairing, the sign of the
 *   rotation and the angle layout are conventions the pages leave open.
 *
 * Entry points:
 *   bfly_prepare, bfly_prepare_hadamard          angles (or H_n) -> coefficient table
 *   bfly_forward, bfly_forward_quant             Q x, fused group quantization
 *   bfly_kron_forward, bfly_kron_forward_wide    (O kron B) x for n = m * nb
 *   bfly_backward, bfly_kron_backward            dX and the angle gradients
 *   bfly_calib_step, bfly_calib_step_weight      one step of learning the angles
 *   bfly_quant_matmul                            y = (Q x)(W Q^T)^T from the codes
 *   bfly_*_bytes, bfly_status_string, bfly_last_hip_error
 *   bfly_forward_quant_noalloc                   bfly_forward_quant with a fixed scratch
 *   bfly_time_next_forward                       kernel-only timing of the next forward
 *
 * Extensions beyond the four calls the pages' problem statement gives
 * (forward, fused forward + quantization, Kronecker forward, backward):
 * the prepared table (`coeffs`, bfly_prepare) that lets fixed angles skip
 * their preparation on every call, the workspace arguments that carry the
 * table when it is prepared per call, and the measurement hook
 * bfly_time_next_forward.  None of them changes what is computed.
 *
 * Conventions common to every call:
 *   - All data pointers are DEVICE pointers owned by the caller, contiguous
 *     row-major with a row stride of n elements (bytes for codes: n*bits/8).
 *     x, y, codes and g/dx must be 16-byte aligned; scales and zeros 2-byte.
 *   - y == x (in place) is allowed, as is dx == g; no other aliasing.
 *   - theta: fp32 angles [log2 n][n/2] on the device.
 *   - coeffs: optional device table prepared from theta by bfly_prepare().
 *     When coeffs is non-NULL, theta is not read (it may be NULL), no
 *     preparation runs and a forward call's workspace is not used (it may
 *     be NULL).  When coeffs is NULL the call first prepares the table from
 *     theta into the caller's workspace: the forward calls then need
 *     workspace_bytes >= bfly_coeff_bytes(n) (16-byte aligned), the other
 *     calls size their workspace with their own *_workspace_bytes query.
 *   - The library allocates no memory in any call: every buffer, scratch
 *     included, comes from the caller (bfly_forward_quant_noalloc uses a
 *     fixed array of the library instead).  Its only state is a fixed-size
 *     per-device cache of launch facts (CU count, resident workgroups per
 *     kernel; filled on first use under a lock), the armed events of
 *     bfly_time_next_forward and the per-thread last HIP error.
 *   - hip_stream: a hipStream_t (NULL = the null stream).  Calls enqueue work
 *     and return; results are valid once the stream is synchronised.
 *   - rows == 0 is a no-op returning BFLY_OK (bfly_backward then writes
 *     zeros to dtheta); the row-data pointers may then be NULL.
 *   - Every argument is validated before any HIP call; a validation failure
 *     returns its code and enqueues nothing.  A failed HIP call returns
 *     BFLY_ERR_HIP; the HIP error code is then available from
 *     bfly_last_hip_error() on the calling thread.
 *   - Supported sizes: n a power of two in [64, 8192] for bfly_forward,
 *     bfly_forward_quant (n = 8192 in two passes), bfly_coeff_bytes,
 *     bfly_prepare and bfly_prepare_hadamard; in [64, 4096] for
 *     bfly_forward_quant_noalloc, bfly_backward and the calibration steps.
 *     Smaller powers of two, and 8192 where it is not listed, return
 *     BFLY_ERR_UNSUPPORTED; for bfly_kron_forward
 *     m in [1, 8] and nb a power of two with m * nb <= 8192, nb in
 *     [256, 4096] for m >= 2 and in [64, 4096] for m = 1; for the wide
 *     forward and the Kronecker backward m in [2, 64], nb in [256, 4096],
 *     m * nb <= 65536.
 *   - Results do not depend on the launch configuration or on the device's
 *     compute-unit count (the angle-gradient reduction order is fixed).
 */
#ifndef BFLY_H
#define BFLY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The two range markers of each enumeration here are no valid value: they
 * make every 32-bit integer a value of the type, so that an out-of-range
 * argument from a caller reaches the library's checks (a dtype or mode is
 * rejected with BFLY_ERR_DTYPE or BFLY_ERR_QUANT) instead of being undefined
 * in C++. */
typedef enum {
    BFLY_OK = 0,
    BFLY_ERR_NULL = 1,        /* a required pointer is NULL                       */
    BFLY_ERR_SIZE = 2,        /* rows < 0, n not a power of two, m*nb mismatch ... */
    BFLY_ERR_DTYPE = 3,       /* dtype not in bfly_dtype                           */
    BFLY_ERR_ALIGN = 4,       /* a pointer is not aligned as stated above          */
    BFLY_ERR_QUANT = 5,       /* bits / group / mode / zeros combination invalid   */
    BFLY_ERR_WORKSPACE = 6,   /* workspace or coefficient buffer too small         */
    BFLY_ERR_UNSUPPORTED = 7, /* a valid size the library does not handle         */
    BFLY_ERR_HIP = 8,         /* a HIP runtime call failed                         */
    BFLY_STATUS_RANGE_LOW_ = -2147483647 - 1,
    BFLY_STATUS_RANGE_HIGH_ = 2147483647
} bfly_status;

typedef enum {
    BFLY_F32 = 0,
    BFLY_BF16 = 1,
    BFLY_DTYPE_RANGE_LOW_ = -2147483647 - 1,
    BFLY_DTYPE_RANGE_HIGH_ = 2147483647
} bfly_dtype;

/* Quantizer modes (WUSH page, technical summary section 2: round-to-nearest
 * with absmax block scaling; ButterflyQuant abstract: 2-bit weights).
 *   BFLY_SYM_ABSMAX : scale = fp16(absmax / qmax), qmax = 2^(bits-1) - 1,
 *                     q = clamp(rne(y / scale), -qmax, qmax), stored as a
 *                     two's-complement bit field.
 *   BFLY_ASYM_MINMAX: scale = fp16((max - min) / (2^bits - 1)),
 *                     zero  = clamp(rne(-min / scale), 0, 2^bits - 1) (an
 *                     integer, stored exactly as fp16),
 *                     q = clamp(rne(y / scale) + zero, 0, 2^bits - 1).
 *   A scale above 65504 saturates to 65504; a zero scale gives zero codes
 *   (and a zero point of 0).  rne = round to nearest, ties to even; the
 *   quantized value is the fp32 y before any bf16 rounding of the output. */
typedef enum {
    BFLY_SYM_ABSMAX = 0,
    BFLY_ASYM_MINMAX = 1,
    BFLY_QMODE_RANGE_LOW_ = -2147483647 - 1,
    BFLY_QMODE_RANGE_HIGH_ = 2147483647
} bfly_qmode;

/* ---- angle preparation ------------------------------------------------- */

/* Bytes of the coefficient table for a butterfly of length n (0 if n is not
 * supported). */
size_t bfly_coeff_bytes(int32_t n);

/* Turn angles theta (device fp32 [log2 n][n/2]) into the device coefficient
 * table `coeffs` (caller-owned, >= bfly_coeff_bytes(n) bytes, 16-byte
 * aligned).  The table depends only on theta; it stays valid for any number
 * of calls with the same angles.  Passage: ButterflyQuant abstract
 * (continuous Givens rotation angles). */
bfly_status bfly_prepare(const float* theta, int32_t n, void* coeffs, size_t coeff_bytes,
                         void* hip_stream);

/* The Hadamard special case: write into `coeffs` (as for bfly_prepare) the
 * table of H_n, the orthonormal Sylvester-ordered Walsh-Hadamard matrix
 * (entries +-1/sqrt(n), H_n[i][j] = (-1)^popcount(i & j) / sqrt(n)).  It is
 * the butterfly with every angle pi/4 after a fixed diagonal
 * D = diag((-1)^popcount(i)) on the input: H_n = Q(pi/4) D.  The table is
 * computed in fp64 from exact constants (no angles are read) and serves
 * bfly_forward, bfly_forward_quant and bfly_kron_forward (as coeffs or
 * coeffs_b) exactly as a table from bfly_prepare does; bfly_backward takes
 * only tables of bfly_prepare.  Errors: BFLY_ERR_NULL (coeffs NULL),
 * BFLY_ERR_SIZE, BFLY_ERR_WORKSPACE (coeff_bytes too small), BFLY_ERR_ALIGN,
 * BFLY_ERR_HIP.  Passage: ButterflyQuant (the butterfly section: H_n for
 * n = 2^k is a butterfly with particular angles) and its abstract (Hadamard
 * coherence 1/sqrt(n)). */
bfly_status bfly_prepare_hadamard(int32_t n, void* coeffs, size_t coeff_bytes, void* hip_stream);

/* ---- forward ------------------------------------------------------------ */

/* y[r] = Q(theta) x[r] for r < rows.  x_dt, y_dt in {BFLY_F32, BFLY_BF16};
 * bf16 outputs are rounded to nearest even from fp32.  workspace: with
 * coeffs == NULL, >= bfly_coeff_bytes(n) bytes of device scratch that
 * receives the table (BFLY_ERR_NULL if missing, BFLY_ERR_WORKSPACE if
 * smaller); ignored with coeffs.  Its contents on entry do not matter.
 * n = 8192 runs in two passes (stages 0..11 on each half of the row, then
 * stage 12 with the output and quantizer) and always needs a workspace of
 * >= bfly_forward_workspace_bytes(rows, 8192) bytes: the table area, then
 * the rows in fp32 between the passes.  Passage: ButterflyQuant abstract
 * (Q x and W Q^T). */
bfly_status bfly_forward(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                         int64_t rows, int32_t n, const float* theta, const void* coeffs,
                         void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes of a forward call (bfly_forward, bfly_forward_quant) of
 * `rows` rows of length n: bfly_coeff_bytes(n) for n <= 4096 (needed when
 * the table comes from theta), the table area rounded up to 256 bytes plus
 * rows * 8192 * 4 for n = 8192; 0 for sizes the library does not handle. */
size_t bfly_forward_workspace_bytes(int64_t rows, int32_t n);

/* The forward, fused with per-group round-to-nearest quantization of y.
 *   y      : may be NULL (codes only); else [rows][n] of y_dt
 *   codes  : u8 [rows][n*bits/8], element e of a byte group in bits
 *            [bits*e, bits*(e+1)) (little-endian packing)
 *   scales : fp16 bit patterns [rows][n/group]
 *   zeros  : fp16 bit patterns [rows][n/group] for BFLY_ASYM_MINMAX; must be
 *            NULL for BFLY_SYM_ABSMAX
 *   bits   : 2 or 4; group: 8, 16, 32, 64, 128, 256 or 512, dividing n;
 *            groups are runs of `group` consecutive output elements.
 *   workspace, workspace_bytes: as in bfly_forward.
 * Passages: ButterflyQuant abstract (orthogonal transforms applied before
 * quantization), WUSH technical summary section 2 (RTN absmax quantizer). */
bfly_status bfly_forward_quant(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                               uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                               int64_t rows, int32_t n, const float* theta, const void* coeffs,
                               int32_t bits, int32_t group, bfly_qmode mode, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

/* bfly_forward_quant for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation from theta, with the coefficient table
 * prepared into a fixed scratch array inside the library instead of a
 * caller workspace.  Each device the library runs on holds one such array
 * (713 KiB: the table of n = 4096) until the process ends; every call on a
 * device shares it, so calls that overlap on one device (two streams, two
 * threads) race on it and must be serialised by the caller.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Arguments and errors as bfly_forward_quant with theta required (there is
 * no coeffs); n above 4096 returns BFLY_ERR_UNSUPPORTED. */
bfly_status bfly_forward_quant_noalloc(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                                       uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                       int64_t rows, int32_t n, const float* theta, int32_t bits,
                                       int32_t group, bfly_qmode mode, void* hip_stream);

/* Kronecker composite for widths n = m * nb that are not a power of two
 * (duidaima.com write-up, section "butterfly": LLaMA-2-13B's 5120):
 *   y[r] = (O kron B(theta_b)) x[r], index i = a * nb + b (a < m, b < nb):
 *   the butterfly B (angles theta_b [log2 nb][nb/2], or its prepared table
 *   coeffs_b) acts on each segment a, then the dense m x m factor
 *   mix (device fp32, row-major) mixes the segments column by column:
 *   y[a*nb + b] = sum_a' mix[a][a'] z[a'*nb + b].
 * codes == NULL => no quantization (scales and zeros must then be NULL);
 * otherwise as in bfly_forward_quant, with group dividing nb.  workspace:
 * with coeffs_b == NULL, >= bfly_coeff_bytes(nb) bytes (as in
 * bfly_forward). */
bfly_status bfly_kron_forward(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                              uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                              int64_t rows, int32_t m, int32_t nb, const float* theta_b,
                              const void* coeffs_b, const float* mix,
                              int32_t bits, int32_t group, bfly_qmode mode, void* workspace,
                              size_t workspace_bytes, void* hip_stream);

/* Kronecker composites with more segments: the same y[r] = (O kron
 * B(theta_b)) x[r] and optional quantization as bfly_kron_forward, for
 * m in [2, 64] (e.g. 11008 = 43 * 256), nb a power of two in [256, 4096],
 * m * nb <= 65536.  bf16 rows with nb = 256 (e.g. 11008) run in one pass
 * (per row: the mix on the matrix cores into LDS, then the butterfly and
 * the quantizer on each segment); otherwise two passes: v = (O kron I) x in
 * fp32 into `workspace`, then the butterfly with its fused quantizer on the
 * rows * m segments of v ((O kron B) = (I kron B)(O kron I)).  y == x is
 * allowed.  workspace (either way): >=
 * bfly_kron_forward_wide_workspace_bytes(rows, m, nb) bytes of device
 * memory (the table's bytes rounded up to 256, then rows * m * nb * 4),
 * 16-byte aligned, caller-owned.  codes == NULL => no quantization
 * (scales, zeros then NULL); otherwise as in bfly_forward_quant with group
 * dividing nb.  With theta_b (no coeffs_b) the table is prepared into the
 * workspace.  Errors as bfly_kron_forward, plus BFLY_ERR_WORKSPACE.  Passage: ButterflyQuant write-up, section
 * "butterfly" (Kronecker composites for widths that are not powers of
 * two). */
bfly_status bfly_kron_forward_wide(const void* x, bfly_dtype x_dt, void* y, bfly_dtype y_dt,
                                   uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                   int64_t rows, int32_t m, int32_t nb, const float* theta_b,
                                   const void* coeffs_b, const float* mix, int32_t bits,
                                   int32_t group, bfly_qmode mode, void* workspace,
                                   size_t workspace_bytes, void* hip_stream);

size_t bfly_kron_forward_wide_workspace_bytes(int64_t rows, int32_t m, int32_t nb);

/* ---- backward ----------------------------------------------------------- */

/* Gradients for learning the angles (ButterflyQuant abstract: smooth
 * optimisation of the continuous angles; duidaima.com write-up, section
 * "training and results").  Given X and G = dL/dY (device fp32 [rows][n]),
 * with Y = Q(theta) X row by row:
 *   y      : Y (optional, may be NULL)            fp32 [rows][n]
 *   dx     : Q^T G                                fp32 [rows][n]
 *   dtheta : sum over rows of dL/dtheta           fp32 [log2 n][n/2], OVERWRITTEN
 * For the pair (i, j) of stage s, with v that stage's output and g the
 * gradient w.r.t. it, dL/dtheta[s][p] = g_j v_i - g_i v_j.  The row sum is a
 * fixed-order two-pass reduction: bit-identical results from run to run.
 * workspace: device scratch of >= bfly_backward_workspace_bytes(rows, n)
 * bytes, 16-byte aligned; the call allocates nothing. */
bfly_status bfly_backward(const float* x, const float* g, float* y, float* dx, float* dtheta,
                          int64_t rows, int32_t n, const float* theta, const void* coeffs,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

size_t bfly_backward_workspace_bytes(int64_t rows, int32_t n);

/* Gradients of the Kronecker composite y = (O kron B(theta_b)) x (see
 * bfly_kron_forward; O = mix, fixed), for learning theta_b.  Given X and
 * G = dL/dY (device fp32 [rows][m*nb]):
 *   dx       : (O kron B)^T G                   fp32 [rows][m*nb] (may be g)
 *   dtheta_b : sum over rows and segments of dL/dtheta_b, fp32
 *              [log2 nb][nb/2], OVERWRITTEN (zeros when rows == 0)
 * Computed as dL/dz = (O^T kron I) G, then the butterfly backward on the
 * rows * m segments of length nb (z = (I kron B) x per segment), with the
 * same fixed-order reduction as bfly_backward.  For m <= 5 and dx != g the
 * backward kernel forms dL/dz from G's m segments as it loads them (one
 * pass); otherwise a mixing pass writes dL/dz into dx first.  Both give the
 * same bits (dx and dtheta_b).  Sizes: m in [2, 64] (m = 1
 * is the plain butterfly: bfly_backward), nb a power of two in [256, 4096],
 * m * nb <= 65536.  workspace: >= bfly_kron_backward_workspace_bytes(rows, m,
 * nb) bytes of device scratch, 16-byte aligned; the call allocates nothing.
 * Errors as bfly_backward.  Passages: ButterflyQuant write-up, section
 * "butterfly" (the Kronecker composite for widths like 5120) and section
 * "training and results" (the angles are learned by gradient descent). */
bfly_status bfly_kron_backward(const float* x, const float* g, float* dx, float* dtheta_b,
                               int64_t rows, int32_t m, int32_t nb, const float* theta_b,
                               const void* coeffs_b, const float* mix, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

size_t bfly_kron_backward_workspace_bytes(int64_t rows, int32_t m, int32_t nb);

/* ---- one calibration step for the angles --------------------------------- */

/* Settings of bfly_calib_step (readings of the pages: they name the loss
 * terms, not these values). */
typedef struct {
    int32_t bits;       /* quantizer of the reconstruction term: symmetric absmax, 2 or 4 */
    int32_t group;      /* its group size: a power of two in [8, 512] dividing n */
    int32_t bins;       /* histogram bins of the uniformity term, in [2, 32] */
    float lambda_kl;    /* weight of the uniformity term */
    float lr, beta1, beta2, eps;  /* Adam */
} bfly_calib_config;

/* One step of learning the angles on calibration rows X (device fp32
 * [rows][n], rows >= 1): Y = Q(theta) X, the loss
 *   L = sum (y - y^)^2 / N + lambda_kl * KL(p || uniform)
 * (y^ the group quantizer's value of y, held constant; p the distribution of
 * u = y / (group max |y|) on `bins` bins over [-1, 1], linear-interpolation
 * weights, smoothed p' = (p + 1e-6) / (1 + bins 1e-6); the group max held
 * constant), dL/dtheta through the butterfly backward, then one Adam update
 * of theta with state adam_m, adam_v (device fp32 [log2 n][n/2], zero before
 * step 1) and step count `step` (1, 2, ...).  theta, adam_m, adam_v are
 * updated in place; loss (device fp32 [3]) receives L, the reconstruction
 * term and KL, all at the angles before the update.  workspace: >=
 * bfly_calib_workspace_bytes(rows, n) bytes of device scratch, 16-byte
 * aligned; the call allocates nothing.  n: a power of two in [64, 4096].
 * Errors: BFLY_ERR_NULL, BFLY_ERR_SIZE, BFLY_ERR_QUANT (bits, group or bins
 * invalid), BFLY_ERR_WORKSPACE, BFLY_ERR_ALIGN, BFLY_ERR_UNSUPPORTED,
 * BFLY_ERR_HIP.  Passages: ButterflyQuant write-up, section "training and
 * results" (reconstruction loss plus a KL-to-uniform regulariser on the
 * rotated activations) and the ButterflyQuant abstract (uniformity
 * regularisation; gradient-based learning of the angles on calibration
 * samples). */
bfly_status bfly_calib_step(const float* x, int64_t rows, int32_t n, float* theta, float* adam_m,
                            float* adam_v, int32_t step, const bfly_calib_config* cfg,
                            float* loss, void* workspace, size_t workspace_bytes,
                            void* hip_stream);

size_t bfly_calib_workspace_bytes(int64_t rows, int32_t n);

/* Settings of bfly_calib_step_weight (readings: the pages name the loss
 * terms, not these values). */
typedef struct {
    int32_t bits;       /* the weight quantizer: 2 or 4 bits */
    int32_t group;      /* its group size: a power of two in [8, 512] dividing n; also the
                           group whose max |y| normalises the uniformity term's histogram */
    int32_t mode;       /* its bfly_qmode (BFLY_ASYM_MINMAX for W2A16) */
    int32_t bins;       /* histogram bins of the uniformity term: a power of two in [2, 32] */
    float lambda_kl;    /* weight of the uniformity term */
    float lr, beta1, beta2, eps;  /* Adam */
} bfly_calib_weight_config;

/* One step of learning the angles with the layer's output as the
 * reconstruction target (duidaima.com write-up, section "training and
 * results": the quantized model's output should match the original one;
 * ButterflyQuant abstract: computational invariance W x = (W Q^T)(Q x),
 * 2-bit weights).  With Xr = Q(theta) X (rows of X), Wr = W Q^T (rows of
 * W, quantized by the group quantizer of cfg to What):
 *   L = ||Xr What^T - X W^T||^2 / (rows * out) + lambda_kl * KL(Xr),
 * KL the uniformity term of bfly_calib_step on Xr.  The quantizer's
 * rounding passes gradients straight through (What - Wr held constant); as
 * Q is orthogonal, Xr What^T - X W^T = Xr (What - Wr)^T and dL/dtheta is the
 * butterfly backward of X with dL/dXr = 2 (Xr E^T) E / (rows * out) plus the
 * uniformity term's share, E = What - Wr.  The two products run on the
 * matrix cores in fp32.  Then one Adam update of theta (as bfly_calib_step).
 *   x     : device fp32 [rows][n] calibration activations (rows >= 1)
 *   w     : device [out][n] weight rows, w_dt = BFLY_F32 or BFLY_BF16
 *   out   : a multiple of 16 in [16, 65536], out * n * 4 < 4 GiB
 *   n     : a power of two in [64, 4096]
 *   theta, adam_m, adam_v, step, loss: as in bfly_calib_step (loss[0..2] =
 *           L, the output term, KL at the angles before the update)
 *   workspace: >= bfly_calib_step_weight_workspace_bytes(rows, out, n)
 *           bytes of device scratch, 16-byte aligned; the call allocates
 *           nothing.
 * Errors: BFLY_ERR_NULL, BFLY_ERR_DTYPE, BFLY_ERR_SIZE, BFLY_ERR_QUANT
 * (bits, group, mode or bins invalid), BFLY_ERR_UNSUPPORTED (sizes outside
 * the ranges above), BFLY_ERR_WORKSPACE, BFLY_ERR_ALIGN, BFLY_ERR_HIP. */
bfly_status bfly_calib_step_weight(const float* x, int64_t rows, const void* w, bfly_dtype w_dt,
                                   int32_t out, int32_t n, float* theta, float* adam_m,
                                   float* adam_v, int32_t step,
                                   const bfly_calib_weight_config* cfg, float* loss,
                                   void* workspace, size_t workspace_bytes, void* hip_stream);

size_t bfly_calib_step_weight_workspace_bytes(int64_t rows, int32_t out, int32_t n);

/* ---- consumer of the quantized weights ---------------------------------- */

/* y[r][o] = sum_k a[r][k] * w[o][k] for r < rows, o < n_out: the layer
 * output W x = (W Q^T)(Q x) with a = Q x (bf16 activations, e.g. from
 * bfly_forward) and the rows of W Q^T stored as group codes by
 * bfly_forward_quant (W2A16; 4-bit codes are accepted too).  Passages:
 * ButterflyQuant abstract (computational invariance, 2-bit weights) and the
 * ButterflyQuant write-up, section "training and results" (W2A16).
 *   a      : bf16 [rows][k] (a_dt must be BFLY_BF16), 16-byte aligned
 *   codes  : u8 [n_out][k*bits/8], the packing of bfly_forward_quant
 *            (element e of a byte in bits [bits*e, bits*(e+1)); symmetric
 *            codes are two's-complement fields), 16-byte aligned
 *   scales : fp16 bit patterns [n_out][k/group], 2-byte aligned
 *   zeros  : fp16 bit patterns [n_out][k/group] (integers) for
 *            BFLY_ASYM_MINMAX, NULL for BFLY_SYM_ABSMAX
 *   y      : [rows][n_out] of y_dt (BFLY_F32 or BFLY_BF16, rounded to
 *            nearest even from fp32), 16-byte aligned; must not overlap
 *            the inputs
 *   w[o][k] = scale * q (symmetric) or scale * (q - zero) (asymmetric).
 * Arithmetic: sums of a * (q - zero) in fp32 (exact products) over one
 * group, each times its group's scale and added in fp32.  With rows <= 64
 * the group sum is formed as C - zero * S from the fp32 sums C of a * q
 * (q the code as offset binary: a symmetric code plus 2^(bits-1), with
 * that as its zero point) and S of a, over the group.
 * Sizes: bits 2 or 4; k a multiple of 64 in [64, 65536]; group one of 64,
 * 128, 256, 512 dividing k; n_out a positive multiple of 128 with
 * n_out <= 1048576.  rows == 0 is a no-op.  Errors: BFLY_ERR_NULL,
 * BFLY_ERR_SIZE (rows < 0, n_out or k not positive), BFLY_ERR_DTYPE,
 * BFLY_ERR_QUANT (bits, group, mode or zeros invalid), BFLY_ERR_ALIGN,
 * BFLY_ERR_UNSUPPORTED (valid sizes outside the ranges above),
 * BFLY_ERR_HIP. */
bfly_status bfly_quant_matmul(const void* a, bfly_dtype a_dt, const uint8_t* codes,
                              const uint16_t* scales, const uint16_t* zeros, void* y,
                              bfly_dtype y_dt, int64_t rows, int32_t n_out, int32_t k,
                              int32_t bits, int32_t group, bfly_qmode mode, void* hip_stream);

/* ---- diagnostics -------------------------------------------------------- */

const char* bfly_status_string(bfly_status s);

/* The hipError_t of the last failed HIP call on this thread (0 if none). */
int32_t bfly_last_hip_error(void);

/* Kernel-only timing of the fused forward kernel (a measurement hook, not
 * part of the method; an extension of the ABI, see above).  start_event and stop_event are hipEvent_t handles
 * the caller created (timing enabled) and owns.  The next launch of the
 * fused forward kernel in this process, by bfly_forward, bfly_forward_quant,
 * bfly_kron_forward or bfly_kron_forward_wide on any stream, is dispatched
 * with the two events attached to the dispatch itself, so that
 * hipEventElapsedTime(start, stop) is that kernel's own start-to-end time
 * (the span a kernel trace reports), without marker packets on the stream
 * and the dispatch delay after them.  One-shot: that launch disarms it; a
 * call that fails validation launches nothing and leaves it armed.  A second
 * call before the launch replaces the pair; both handles NULL disarms.
 * Returns BFLY_ERR_NULL if exactly one handle is NULL (nothing changes);
 * makes no HIP call. */
bfly_status bfly_time_next_forward(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* BFLY_H */
