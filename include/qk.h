/*
 * qk.h -- C ABI of libqk, an MI355X (gfx950) W8A8 INT8 linear layer.
 *
 * The layer (all steps on the GPU, in HIP kernels of this library):
 *   1. per-token dynamic INT8 quantization of the activations, optionally of
 *      silu(gate) * up;
 *   2. an INT8 x INT8 product accumulated in INT32;
 *   3. a dequant epilogue  out = acc * scale_a[row] * scale_b[col] * output_scale.
 * and the same layer with float8_e4m3fn codes (per-token FP8 quantization
 * with an optional scale bound, an FP8 x FP8 product accumulated in
 * binary32, the same epilogue).
 *
 * Sources, cited by page title and section:
 *   "16. Deploying Custom Kernels", C++ Kernel Interface: the GEMM problem
 *     statement (GemmConfig: m, n, k, int8 a and b, int32 c, fp32 scale_a and
 *     scale_b, float output_scale, stream) and a status return;
 *     Python Bindings: the argument order of the flat call.
 *   "Skill: Write an INT8 Quantized Kernel", Inputs the agent should gather
 *     first: symmetric [-127, 127] codes with zero point 0, INT32
 *     accumulation, per-token and per-channel scales, fp32/fp16 output,
 *     row- or column-major weights.
 *   "KV-cache kernels", 02 Scales and dequantization: int8 products
 *     accumulate in int32, then acc * a_scale * b_scale.
 *   "kernels: fused silu_and_mul + dynamic per-token FP8 quantization",
 *     Purpose and Algorithm: one scale per token from the row absmax,
 *     scale = max(absmax, 1e-12) / qmax, optionally of silu(gate) * up.
 *   "dynquant-kernels", Variants: an ABI number checked by the loader.
 *
 * Conventions (every function):
 *   - Pointers to tensors are DEVICE pointers on the current HIP device;
 *     every tensor is dense and row-major.  The caller allocates and owns all
 *     memory; the library allocates nothing and keeps no pointer after a call
 *     returns.  Outputs must not alias inputs.
 *   - Work is enqueued on `stream` (0 = the null stream) and runs
 *     asynchronously; a fault during execution surfaces at the caller's next
 *     synchronisation.
 *   - The return value is a status: QK_OK (0) on success; QK_ERR_* (>= 1000)
 *     for an argument error detected on the host before anything is
 *     enqueued; otherwise the hipError_t of a failed launch.  Nothing aborts
 *     and no C++ exception crosses this interface.
 *   - Dimensions are int; m == 0 or n == 0 is a successful no-op.
 */
#ifndef QK_H
#define QK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QK_ABI_VERSION 7

/* element types */
#define QK_F32 0
#define QK_BF16 1
#define QK_F16 2

/* weight layouts */
#define QK_B_KN 0 /* b is [k][n], n contiguous (the default) */
#define QK_B_NK 1 /* b is [n][k], k contiguous */

/* GEMM kernel choice for qk_gemm_i8_scaled_ex */
#define QK_KERNEL_AUTO 0 /* by shape: decode GEMV for m <= 8, MFMA tiles otherwise */
#define QK_KERNEL_MFMA 1 /* LDS-tiled INT8 MFMA kernel, any m */
#define QK_KERNEL_GEMV 2 /* split-K decode GEMV: m <= 16, [k][n] weight (per launch of up
                          * to 8 rows: dot products for 1-3, matrix cores for 4-8) */

/* status codes */
#define QK_OK 0
#define QK_ERR_INVALID_VALUE 1001 /* negative size, NULL pointer, unknown enum */
#define QK_ERR_UNSUPPORTED 1002   /* a size or alignment this library does not handle */
#define QK_ERR_WORKSPACE 1003     /* workspace missing, misaligned or too small */
#define QK_ERR_SCRATCH_LIMIT 1004 /* qk_linear_w8a8_noalloc: more scratch needed than it has */

/* Largest reduction length accepted: 131071 * 128 * 128 < 2^31, so no int32
 * accumulator can overflow even for -128 operands ("Skill: Write an INT8
 * Quantized Kernel", Inputs: INT32 accumulation is mandatory). */
#define QK_MAX_K 131071

/* Compiled-in ABI number.  A loader must refuse the library when it differs
 * from the number it was written for ("dynquant-kernels", Variants). */
int qk_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *qk_status_string(int status);

/* Static text: code-object architectures, HIP version, ABI number
 * (after "dynquant-kernels", Diagnosing an install). */
const char *qk_build_info(void);

/*
 * Per-token dynamic INT8 quantization ("kernels: fused silu_and_mul + dynamic
 * per-token FP8 quantization", Algorithm, with the symmetric [-127, 127]
 * range of "Skill: Write an INT8 Quantized Kernel", Inputs):
 *   scale[i] = max(max_j |x[i][j]|, 1e-12f) / 127       (binary32 division)
 *   q[i][j]  = clamp(rint(x[i][j] / scale[i]), -127, 127) (binary32 division,
 *                                                          ties to even)
 *   x       [m][k] of x_dtype (QK_F32, QK_BF16 or QK_F16), read only.
 *   q       [m][k] int8, written.
 *   scale   [m] float, written.
 * Any k >= 0 (k == 0 gives scale = 1e-12f / 127).  Errors: m or k negative,
 * m*k > 2^62, NULL pointer with m*k > 0 (QK_ERR_INVALID_VALUE); unknown
 * dtype (QK_ERR_INVALID_VALUE).
 */
int qk_quant_per_token(int m, int k, const void *x, int x_dtype, int8_t *q, float *scale,
                       hipStream_t stream);

/*
 * silu(gate) * up followed by per-token INT8 quantization, one pass over h
 * ("kernels: fused silu_and_mul + dynamic per-token FP8 quantization",
 * Purpose and Algorithm):
 *   g = h[i][j], u = h[i][d + j];  a[i][j] = (g / (1 + exp(-g))) * u  (binary32)
 *   then scale[i] and q[i][j] as qk_quant_per_token on a.
 *   exp is the library's fixed binary32 algorithm (reduction by ln 2, degree-7
 *   Taylor polynomial with fused multiply-adds, scaling by 2^n; inputs above
 *   88 give +inf, below -87 give 0), so results are reproducible bit for bit.
 *   h       [m][2d] of h_dtype, gate = first half of each row, up = second.
 *   q       [m][d] int8;  scale [m] float.
 * Errors as qk_quant_per_token.
 */
int qk_silu_mul_quant_per_token(int m, int d, const void *h, int h_dtype, int8_t *q,
                                float *scale, hipStream_t stream);

/*
 * silu(gate) * up alone, in binary32, with exactly the arithmetic of
 * qk_silu_mul_quant_per_token before its quantization ("kernels: fused
 * silu_and_mul + dynamic per-token FP8 quantization", Purpose: the
 * silu_and_mul activation):
 *   out[i][j] = (g / (1 + exp(-g))) * u,  g = h[i][j], u = h[i][d + j]
 *   h    [m][2d] of h_dtype (QK_F32, QK_BF16 or QK_F16), gate | up.
 *   out  [m][d] float, written.
 * Any alignment.  Errors: m or d negative, NULL pointer with m*d > 0, unknown
 * dtype (QK_ERR_INVALID_VALUE); 2d above INT_MAX (QK_ERR_UNSUPPORTED).
 */
int qk_silu_mul(int m, int d, const void *h, int h_dtype, float *out, hipStream_t stream);

/* Bytes of workspace qk_gemm_i8_scaled / qk_linear_w8a8 need for this shape
 * (0 if none).  The decode kernel (m <= 16) keeps one 64-bit word per output
 * element of a row group there, holding the exact split-K partial sum and the
 * number of contributions so far.  The tiled kernel uses it when the output
 * has fewer than 128 tiles of 256 x 128 (n % 16 == 0, k % 128 == 0,
 * k >= 2048) and the k time saved outweighs the partial sums'
 * round trip: it then splits k, stores each slice's INT32 partial sums there
 * and adds them in a second launch (exact, the same bits on every run); with
 * a smaller workspace, or none, it runs unsplit. */
size_t qk_gemm_workspace_size(int m, int n, int k);

/*
 * Prepares a workspace for the calls that take one: enqueues, on `stream`, a
 * kernel that sets all `workspace_bytes` bytes to zero (a kernel, not a
 * memset, so that the call may be captured in a HIP graph).  The caller
 * allocates and owns the workspace ("16. Deploying Custom Kernels", C++
 * Kernel Interface: caller-owned buffers, a status return); the library
 * keeps it zero from then on:
 *   - call it once on a new workspace before its first use (memory from an
 *     allocator holds arbitrary bytes);
 *   - every call that uses the workspace and returns QK_OK leaves it all
 *     zeros when its work completes, so later calls issued in order on one
 *     stream need no further initialization;
 *   - after a call returns a HIP launch error (a status below 1000 other
 *     than QK_OK), part of its work may have run: call this again before the
 *     workspace is reused.  Host-detected errors (QK_ERR_*) enqueue nothing
 *     and leave the workspace as it was.
 *   workspace        device memory, 256-byte aligned (NULL only with 0 bytes).
 *   workspace_bytes  any size; usually qk_gemm_workspace_size(m, n, k).
 * Errors: NULL with workspace_bytes > 0 (QK_ERR_INVALID_VALUE); misaligned
 * (QK_ERR_WORKSPACE).
 */
int qk_workspace_init(void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * INT8 GEMM with INT32 accumulation and the dequant epilogue
 * ("16. Deploying Custom Kernels", C++ Kernel Interface and Python Bindings
 * for the first nine arguments; "KV-cache kernels", 02 Scales and
 * dequantization for the epilogue):
 *   acc[i][j] = sum_t a[i][t] * B(t, j)              (exact, INT32)
 *   c[i][j]   = acc[i][j]                            (if c != NULL; raw)
 *   out[i][j] = (float)acc * scale_a[i] * scale_b[j] * output_scale
 *                                                    (if out != NULL; binary32
 *                                                    arithmetic, stored as fp32
 *                                                    or bf16 rounded to nearest even)
 *   a        [m][k] int8 (the quantized activations).
 *   b        [k][n] int8 (QK_B_KN) or [n][k] int8 (QK_B_NK).
 *   c        [m][n] int32 or NULL.
 *   scale_a  [m] float (per token), scale_b [n] float (per output channel);
 *            both may be NULL only when out is NULL.
 *   out      [m][n] of out_dtype (QK_F32 or QK_BF16) or NULL; c and out may
 *            not both be NULL.
 *   workspace / workspace_bytes: device memory of at least
 *            qk_gemm_workspace_size(m, n, k) bytes, 256-byte aligned, set up
 *            by qk_workspace_init before its first use; every successful
 *            call returns it to all zeros when it completes, so one buffer
 *            serves all calls issued in order on a stream.  Calls that can
 *            run at the same time must not share one.  May be NULL when the
 *            size is 0; otherwise a missing or short workspace is
 *            QK_ERR_WORKSPACE on the decode path, while the tiled GEMM then
 *            runs unsplit.
 * Requirements: 0 <= k <= QK_MAX_K and k % 16 == 0; a, b 16-byte aligned;
 * for the tiled (m > 8) kernel m*k and n*k below 2^32 (QK_ERR_UNSUPPORTED
 * otherwise).  k == 0 gives acc = 0.
 */
int qk_gemm_i8_scaled(int m, int n, int k, const int8_t *a, const int8_t *b, int32_t *c,
                      const float *scale_a, const float *scale_b, float output_scale, void *out,
                      int out_dtype, int b_layout, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* As qk_gemm_i8_scaled with an explicit kernel choice (QK_KERNEL_*), so that
 * both kernels can be checked at any shape.  QK_KERNEL_GEMV requires m <= 16
 * and a [k][n] weight (QK_ERR_UNSUPPORTED otherwise). */
int qk_gemm_i8_scaled_ex(int m, int n, int k, const int8_t *a, const int8_t *b, int32_t *c,
                         const float *scale_a, const float *scale_b, float output_scale,
                         void *out, int out_dtype, int b_layout, void *workspace,
                         size_t workspace_bytes, int kernel, hipStream_t stream);

/*
 * The whole layer: per-token quantization of x, the INT8 GEMM and the
 * dequant epilogue (same arithmetic as qk_quant_per_token followed by
 * qk_gemm_i8_scaled with scale_a = the per-token scales).
 *   x        [m][k] of x_dtype (QK_F32, QK_BF16, QK_F16).
 *   b        [k][n] (QK_B_KN) or [n][k] (QK_B_NK) int8; scale_b [n] float.
 *   out      [m][n] of out_dtype (QK_F32 or QK_BF16), or NULL.
 *   c_out    [m][n] int32 raw accumulators, or NULL; c_out and out may not
 *            both be NULL.
 *   q_out, scale_out: [m][k] int8 codes and [m] scales.  Optional when the
 *            call runs as one fused decode launch (m <= 8, [k][n] weight,
 *            x 16-byte aligned, kernel AUTO or GEMV); then they receive the
 *            codes and scales if given.  Required otherwise: they hold the
 *            intermediate between the two launches.
 *   workspace / workspace_bytes: as for qk_gemm_i8_scaled (used by the
 *            fused decode launch, and by the tiled GEMM to split k).
 *   kernel   QK_KERNEL_AUTO, QK_KERNEL_GEMV (fused, m <= 16) or
 *            QK_KERNEL_MFMA (quantization launch + tiled GEMM).
 * Requirements and errors as qk_quant_per_token and qk_gemm_i8_scaled.
 */
int qk_linear_w8a8(int m, int n, int k, const void *x, int x_dtype, const int8_t *b,
                   const float *scale_b, float output_scale, void *out, int out_dtype,
                   int b_layout, int8_t *q_out, float *scale_out, int32_t *c_out,
                   void *workspace, size_t workspace_bytes, int kernel, hipStream_t stream);

/* Bytes of device scratch the library holds per GPU for
 * qk_linear_w8a8_noalloc (16 MiB). */
#define QK_SCRATCH_BYTES 16777216

/*
 * qk_linear_w8a8 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same layer and arguments without the workspace: in its place the call
 * uses QK_SCRATCH_BYTES of static device memory inside the library (one copy
 * per GPU, held until the process ends), and it calls no allocator.  The
 * caller still passes x, b, scale_b and the outputs (and q_out / scale_out
 * where qk_linear_w8a8 requires them).
 *   - The fused decode launch needs 64 bytes of scratch per output column:
 *     n > QK_SCRATCH_BYTES / 64 = 262144 on that path is QK_ERR_SCRATCH_LIMIT
 *     (nothing is enqueued).  The tiled GEMM splits k only when its partial
 *     sums fit in the scratch and otherwise runs unsplit; results are the
 *     same bits either way.
 *   - All calls on one GPU share its scratch, which keeps the last call's
 *     contents (all zeros after a successful call): calls that can overlap on
 *     one GPU (other streams, other host threads) race and must be ordered by
 *     the caller.  The first call on a GPU, and the first after a call that
 *     returned a HIP launch error, clear the scratch with a kernel on `stream`
 *     before using it.
 * Requirements and errors otherwise as qk_linear_w8a8.
 */
int qk_linear_w8a8_noalloc(int m, int n, int k, const void *x, int x_dtype, const int8_t *b,
                           const float *scale_b, float output_scale, void *out, int out_dtype,
                           int b_layout, int8_t *q_out, float *scale_out, int32_t *c_out,
                           int kernel, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* FP8 path: float8_e4m3fn activations and weights                     */
/* ------------------------------------------------------------------ */
/*
 * float8_e4m3fn (the page's format): sign, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448,
 * subnormals m * 2^-9.  Codes are passed as uint8_t bytes.
 */

/*
 * Per-token dynamic FP8 quantization ("kernels: fused silu_and_mul + dynamic
 * per-token FP8 quantization", Algorithm: scale from the row absmax over
 * fp8_max, optionally clamped by scale_ub):
 *   scale[i] = max(max_j |x[i][j]|, 1e-12f) / 448          (binary32 division)
 *              then min(scale[i], scale_ub) when scale_ub > 0
 *   q[i][j]  = e4m3fn(x[i][j] / scale[i])   (binary32 quotient; nearest,
 *              ties to even; saturating at +-448; the sign of zero kept)
 *   x        [m][k] of x_dtype (QK_F32, QK_BF16 or QK_F16), read only.
 *   scale_ub upper bound on the scale; 0 or negative means none.
 *   q        [m][k] codes, written;  scale [m] float, written.
 * Errors as qk_quant_per_token; a NaN scale_ub is QK_ERR_INVALID_VALUE.
 */
int qk_quant_per_token_fp8(int m, int k, const void *x, int x_dtype, float scale_ub, uint8_t *q,
                           float *scale, hipStream_t stream);

/*
 * silu(gate) * up followed by per-token FP8 quantization, one pass over h
 * (the same page, Purpose and Algorithm; silu exactly as in
 * qk_silu_mul_quant_per_token).
 *   h [m][2d] of h_dtype (gate | up);  q [m][d] codes;  scale [m] float.
 * Errors as qk_quant_per_token_fp8.
 */
int qk_silu_mul_quant_per_token_fp8(int m, int d, const void *h, int h_dtype, float scale_ub,
                                    uint8_t *q, float *scale, hipStream_t stream);

/*
 * FP8 GEMM with binary32 accumulation and the dequant epilogue (the FP8
 * codes above fed to the scaled GEMM of "16. Deploying Custom Kernels", C++
 * Kernel Interface; epilogue of "KV-cache kernels", 02 Scales and
 * dequantization):
 *   acc[i][j] = sum_t value(a[i][t]) * value(B(t, j))  (matrix-core binary32
 *               accumulation: every product exact, sums rounded per 128-deep
 *               step or finer, so acc is not bit-reproducible across
 *               implementations)
 *   c[i][j]   = acc                                 (if c != NULL; binary32)
 *   out[i][j] = (acc * scale_a[i]) * (scale_b[j] * output_scale)
 *               (if out != NULL; binary32, stored as fp32 or bf16 RNE)
 *   a [m][k] codes; b [k][n] (QK_B_KN) or [n][k] (QK_B_NK) codes;
 *   scale_a [m], scale_b [n] float (NULL only when out is NULL);
 *   c [m][n] float or NULL; out [m][n] of out_dtype or NULL (not both NULL).
 * Requirements: 0 <= k <= QK_MAX_K, k % 16 == 0, a and b 16-byte aligned,
 * m*k and n*k below 2^32 (QK_ERR_UNSUPPORTED otherwise).  No workspace.
 * NaN codes propagate.
 */
int qk_gemm_fp8_scaled(int m, int n, int k, const uint8_t *a, const uint8_t *b, float *c,
                       const float *scale_a, const float *scale_b, float output_scale, void *out,
                       int out_dtype, int b_layout, hipStream_t stream);

/*
 * The FP8 layer: qk_quant_per_token_fp8 of x into q_out / scale_out, then
 * qk_gemm_fp8_scaled of those codes with the weight (two launches on
 * `stream`).
 *   x [m][k] of x_dtype;  b [k][n] or [n][k] codes;  scale_b [n] float;
 *   out [m][n] of out_dtype;  q_out [m][k] (16-byte aligned) and
 *   scale_out [m]: required, they hold the codes and scales.
 * Requirements and errors as the two calls.
 */
int qk_linear_fp8(int m, int n, int k, const void *x, int x_dtype, float scale_ub,
                  const uint8_t *b, const float *scale_b, float output_scale, void *out,
                  int out_dtype, int b_layout, uint8_t *q_out, float *scale_out,
                  hipStream_t stream);

/* ------------------------------------------------------------------ */
/* INT8 GEMM with per-group weight scales                              */
/* ------------------------------------------------------------------ */
/*
 * The weight carries one scale per group of `group` consecutive k of each
 * output column ("KV-cache kernels", 02 Scales and dequantization and 03
 * Where scales come from: one scale per group of 64-128 channels, the
 * accuracy lever against outlier channels), so the scale applies to each
 * group's integer partial sum before the groups are added:
 *   P_g[i][j] = sum_{t in group g} a[i][t] * B(t, j)          (exact, INT32)
 *   acc[i][j] = sum_g scale_b[g][j] * P_g[i][j]               (binary32:
 *               each P_g converted exactly, one fused multiply-add per group)
 *   c[i][j]   = acc                                 (if c != NULL; binary32)
 *   out[i][j] = (acc * scale_a[i]) * output_scale   (if out != NULL; fp32 or
 *               bf16 rounded to nearest even)
 *   a [m][k] int8; b [k][n] (QK_B_KN) or [n][k] (QK_B_NK) int8;
 *   scale_b [k / group][n] float (n contiguous); scale_a [m] float (NULL
 *   only when out is NULL); c [m][n] float or NULL; out [m][n] of out_dtype
 *   or NULL (not both NULL).
 * Requirements: group 64 or 128 and k a multiple of it, k <= QK_MAX_K, a and
 * b 16-byte aligned, m*k and n*k below 2^32 (QK_ERR_UNSUPPORTED otherwise).
 * No workspace.
 */
int qk_gemm_i8_grouped(int m, int n, int k, int group, const int8_t *a, const int8_t *b, float *c,
                       const float *scale_a, const float *scale_b, float output_scale, void *out,
                       int out_dtype, int b_layout, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* MoE grouped GEMM                                                     */
/* ------------------------------------------------------------------ */
/* Largest expert count of one qk_moe_gemm_i8_scaled call. */
#define QK_MOE_MAX_EXPERTS 256

/*
 * The INT8 GEMM and dequant epilogue for all experts of a mixture-of-experts
 * layer in one launch ("dynquant-kernels", What is in here: MoE grouped GEMM,
 * one launch for all experts, not one per expert):
 *   rows [expert_offsets[e], expert_offsets[e + 1]) of a are expert e's;
 *   for each such row i:  acc[i][j] = sum_t a[i][t] * B_e(t, j)   (exact, INT32)
 *                         out[i][j] = ((float)acc * scale_a[i]) *
 *                                     (scale_b[e][j] * output_scale)
 *   c[i][j] = acc (if c != NULL).
 *   expert_offsets  DEVICE array of experts + 1 int, nondecreasing, [0] = 0,
 *                   [experts] = m (the routing's row counts as prefix sums).
 *                   Values are clamped to [0, m] inside the kernel: invalid
 *                   offsets give unspecified results but no access out of
 *                   bounds.  Rows outside every expert's range are not written.
 *   a        [m][k] int8 codes, rows grouped by expert.
 *   b        [experts][k][n] (QK_B_KN) or [experts][n][k] (QK_B_NK) int8.
 *   scale_a  [m] float;  scale_b [experts][n] float (both may be NULL only
 *            when out is NULL).
 *   c        [m][n] int32 or NULL;  out [m][n] of out_dtype or NULL (not both).
 * Requirements: 1 <= experts <= QK_MOE_MAX_EXPERTS, k % 16 == 0, a and b
 * 16-byte aligned, m*k and n*k below 2^32.  No workspace; the grid is
 * sized from m and experts, so the call needs no host copy of the offsets.
 */
int qk_moe_gemm_i8_scaled(int experts, int m, int n, int k, const int *expert_offsets,
                          const int8_t *a, const int8_t *b, int32_t *c, const float *scale_a,
                          const float *scale_b, float output_scale, void *out, int out_dtype,
                          int b_layout, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Static (per-tensor) quantization                                    */
/* ------------------------------------------------------------------ */
/*
 * Quantization with one pre-calibrated scale for the whole tensor ("kernels:
 * fused silu_and_mul + dynamic per-token FP8 quantization", Purpose:
 * silu_and_mul_quant takes a global scale), read from DEVICE memory:
 *   INT8:  q[i][j] = clamp(rint(x[i][j] / *scale), -127, 127)
 *   FP8:   q[i][j] = e4m3fn(x[i][j] / *scale)   (nearest even, saturating)
 * (binary32 quotient; the _silu_mul_ forms quantize silu(gate) * up of
 * h [m][2d] as qk_silu_mul_quant_per_token does).
 *   scale  one float on the device, > 0 (not checked; a zero or negative
 *          scale gives unspecified codes).
 * Errors as qk_quant_per_token.
 */
int qk_quant_static(int m, int k, const void *x, int x_dtype, const float *scale, int8_t *q,
                    hipStream_t stream);
int qk_silu_mul_quant_static(int m, int d, const void *h, int h_dtype, const float *scale,
                             int8_t *q, hipStream_t stream);
int qk_quant_static_fp8(int m, int k, const void *x, int x_dtype, const float *scale, uint8_t *q,
                        hipStream_t stream);
int qk_silu_mul_quant_static_fp8(int m, int d, const void *h, int h_dtype, const float *scale,
                                 uint8_t *q, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Asymmetric (zero-point) activations                                 */
/* ------------------------------------------------------------------ */
/* Largest k of the asymmetric GEMM: the zero-point term keeps the INT32
 * result within range (2 * 65535 * 128 * 127 < 2^31). */
#define QK_MAX_K_ASYM 65535

/*
 * Per-token asymmetric INT8 quantization ("Skill: Write an INT8 Quantized
 * Kernel", Inputs: the asymmetric alternative, a nonzero zero point):
 *   lo = min(min_j x[i][j], 0), hi = max(max_j x[i][j], 0)
 *   scale[i]      = max(hi - lo, 1e-12f) / 255                 (binary32)
 *   zero_point[i] = clamp(rint(-lo / scale[i]) - 128, -128, 127)
 *   q[i][j]       = clamp(rint(x[i][j] / scale[i]) + zero_point[i], -128, 127)
 * so x ~ (q - zero_point) * scale, and 0 has the exact code zero_point.
 *   q [m][k] int8, scale [m] float, zero_point [m] int32 (all written).
 * Errors as qk_quant_per_token (NULL zero_point with m > 0 is invalid).
 */
int qk_quant_per_token_asym(int m, int k, const void *x, int x_dtype, int8_t *q, float *scale,
                            int32_t *zero_point, hipStream_t stream);

/* Column sums of an INT8 weight, wsum[j] = sum_t B(t, j) (int32), for the
 * zero-point term of qk_gemm_i8_asym; computed once per weight.
 * b [k][n] (QK_B_KN) or [n][k] (QK_B_NK); wsum [n]. */
int qk_weight_colsum(int k, int n, const int8_t *b, int b_layout, int32_t *wsum,
                     hipStream_t stream);

/*
 * INT8 GEMM of asymmetric activations with the dequant epilogue:
 *   acc[i][j] = sum_t (a[i][t] - zero_point[i]) * B(t, j)
 *             = sum_t a[i][t] * B(t, j) - zero_point[i] * wsum[j]   (exact INT32)
 *   c[i][j]   = acc (if c != NULL)
 *   out[i][j] = ((float)acc * scale_a[i]) * (scale_b[j] * output_scale)
 *   zero_point [m] int32, wsum [n] int32 = qk_weight_colsum of b; other
 *   arguments as qk_gemm_i8_scaled (the tiled kernel for every m).
 * Requirements: 0 <= k <= QK_MAX_K_ASYM, k % 16 == 0, a and b 16-byte
 * aligned, m*k and n*k below 2^32.
 */
int qk_gemm_i8_asym(int m, int n, int k, const int8_t *a, const int32_t *zero_point,
                    const int8_t *b, const int32_t *wsum, int32_t *c, const float *scale_a,
                    const float *scale_b, float output_scale, void *out, int out_dtype,
                    int b_layout, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QK_H */
