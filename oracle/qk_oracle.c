/*
 * CPU oracle for the symmetric W8A8 INT8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is loaded by the test suite, by the
 * package smoke check and by the benchmark's CPU-baseline leg, and by nothing
 * else.  It shares no code, header, table or constant with the GPU library;
 * the two are written independently from the same source pages.
 *
 * It is deliberately plain: straight loops, one step per statement, in the
 * order the pages state the method, so that a reader can check it by eye.
 * OpenMP only splits independent rows across threads; no step is blocked,
 * fused or reordered.
 *
 * Sources (cited by page title and section):
 *   [GEMM-IF]  "16. Deploying Custom Kernels", C++ Kernel Interface -- the
 *              problem statement: m, n, k, int8 A and B, int32 C, fp32
 *              per-row scale_a, per-column scale_b, scalar output_scale.
 *   [SKILL]    "Skill: Write an INT8 Quantized Kernel", Inputs the agent
 *              should gather first -- symmetric range [-127, 127] with zero
 *              point 0; INT32 accumulation is mandatory; per-token and
 *              per-channel granularity; fp32 or fp16 output after dequant.
 *   [DAY25]    "KV-cache kernels" (a quantization lesson), 02 Scales and
 *              dequantization -- int8 dot products accumulate in int32 and
 *              the result is multiplied by the activation and weight scales.
 *   [DAY25-G]  the same lesson, 02 Scales and dequantization and 03 Where
 *              scales come from -- one weight scale per small group of
 *              channels (every 64-128), applied after the load; here the
 *              groups run along the reduction dimension k, so a group's
 *              integer partial sum is scaled before the groups are added.
 *   [PR-S]     the same page, Purpose: silu_and_mul_quant quantizes with one
 *              pre-calibrated (static, per-tensor) scale.
 *   [ASYM]     "Skill: Write an INT8 Quantized Kernel", Inputs -- the
 *              asymmetric alternative to the symmetric range: a nonzero zero
 *              point.  Reading: per token, the range [min(row min, 0),
 *              max(row max, 0)] maps onto [-128, 127].
 *   [PR]       "kernels: fused silu_and_mul + dynamic per-token FP8
 *              quantization", Purpose and Algorithm -- one scale per token
 *              from the row absmax, scale = max(absmax, 1e-12) / qmax, the
 *              value quantized is silu(gate) * up.
 *
 * Precision.  Quantization and the SiLU gate run in IEEE binary32: their
 * results decide integer codes, and the per-token scale is an fp32 value in
 * the interface [GEMM-IF].  The integer product is exact (int64 accumulation,
 * range-checked against int32).  The dequant epilogue is evaluated in
 * binary64 as the reference value an fp32/bf16 result is compared against.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - x / scale is a true IEEE binary32 division (not a reciprocal product),
 *     rounded to an integer with round-half-to-even, then clamped to +-127.
 *   - the 1e-12 guard is the binary32 value nearest 1e-12, applied to the
 *     absmax before the division by 127.
 *   - silu(g) = g / (1 + exp(-g)) with exp evaluated by the fixed binary32
 *     algorithm spec_expf below (Cody-Waite reduction by ln 2, degree-7
 *     Taylor polynomial in Horner form with fused multiply-adds, scaling by
 *     2^n); every other step is one correctly rounded binary32 operation.
 *   - gate is the first half of each row of H, up the second half.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared
 * (-ffp-contract=off: no multiply-add is fused unless written as fmaf).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F16 2

#define OR_B_KN 0 /* weight stored [k][n], n contiguous */
#define OR_B_NK 1 /* weight stored [n][k], k contiguous */

/* ------------------------------------------------------------------ */
/* Step 0: widen the input element to binary32 (exact for all three).  */
/* ------------------------------------------------------------------ */

static float widen_bf16(uint16_t bits)
{
    /* bfloat16 is the upper half of a binary32 word. */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float widen_f16(uint16_t bits)
{
    /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
    int sign = bits >> 15;
    int e = (bits >> 10) & 31;
    int f = bits & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return (float)(sign ? -v : v);
}

int or_widen(int dtype, int64_t count, const void *src, float *dst)
{
    if (dtype == OR_F32) {
        memcpy(dst, src, (size_t)count * sizeof(float));
        return 0;
    }
    if (dtype != OR_BF16 && dtype != OR_F16)
        return 1;
    const uint16_t *s = (const uint16_t *)src;
    for (int64_t i = 0; i < count; ++i)
        dst[i] = dtype == OR_BF16 ? widen_bf16(s[i]) : widen_f16(s[i]);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Steps 1-3: dynamic per-token symmetric quantization [PR], [SKILL].   */
/* ------------------------------------------------------------------ */

/* x: [m][k] binary32, q: [m][k] int8, scale: [m] binary32. */
void or_quant_rows(int64_t m, int64_t k, const float *x, int8_t *q, float *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        const float *row = x + i * k;

        /* 1. row absmax (exact: max is order independent) */
        float amax = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            float a = fabsf(row[j]);
            if (a > amax)
                amax = a;
        }

        /* 2. scale = max(absmax, 1e-12) / 127 */
        float guarded = fmaxf(amax, 1e-12f);
        float s = guarded / 127.0f;
        scale[i] = s;

        /* 3. code = clamp(rint(x / scale), -127, 127) */
        for (int64_t j = 0; j < k; ++j) {
            float ratio = row[j] / s;
            float r = nearbyintf(ratio); /* default rounding mode: to nearest, ties to even */
            if (r > 127.0f)
                r = 127.0f;
            if (r < -127.0f)
                r = -127.0f;
            q[i * k + j] = (int8_t)r;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Step 0': silu(gate) * up [PR], with the binary32 exp spec.           */
/* ------------------------------------------------------------------ */

/* Constants of spec_expf, each the binary32 value nearest the quantity named. */
static const float SPEC_LOG2E = 0x1.715476p+0f;      /* 1 / ln 2 */
static const float SPEC_LN2_HI = 0x1.62e400p-1f;     /* 0.693145751953125, ln 2 cut to 16 bits */
static const float SPEC_LN2_LO = 0x1.7f7d1cp-20f;    /* ln 2 - SPEC_LN2_HI */
static const float SPEC_TAYLOR[8] = {                /* 1 / j! for j = 0..7 */
    0x1.000000p+0f, 0x1.000000p+0f, 0x1.000000p-1f,  0x1.555556p-3f,
    0x1.555556p-5f, 0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f,
};

float or_spec_expf(float x)
{
    if (x > 88.0f)
        return INFINITY;
    if (x < -87.0f)
        return 0.0f;
    float n = nearbyintf(x * SPEC_LOG2E);  /* x = n ln2 + r */
    float r = fmaf(-n, SPEC_LN2_HI, x);
    r = fmaf(-n, SPEC_LN2_LO, r);
    float p = SPEC_TAYLOR[7];              /* e^r by Horner's rule */
    for (int j = 6; j >= 0; --j)
        p = fmaf(p, r, SPEC_TAYLOR[j]);
    return ldexpf(p, (int)n);              /* exact: the result is a normal number */
}

void or_spec_taylor(float *out8)
{
    for (int j = 0; j < 8; ++j)
        out8[j] = SPEC_TAYLOR[j];
}

void or_spec_reduction_constants(float *out3)
{
    out3[0] = SPEC_LOG2E;
    out3[1] = SPEC_LN2_HI;
    out3[2] = SPEC_LN2_LO;
}

void or_expf_array(int64_t count, const float *x, float *y)
{
    for (int64_t i = 0; i < count; ++i)
        y[i] = or_spec_expf(x[i]);
}

/* h: [m][2d] binary32 with gate = h[:, :d], up = h[:, d:]; out: [m][d]. */
void or_silu_mul(int64_t m, int64_t d, const float *h, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < d; ++j) {
            float g = h[i * 2 * d + j];
            float u = h[i * 2 * d + d + j];
            float e = or_spec_expf(-g);
            float t = 1.0f + e;
            float sg = g / t; /* silu(g) = g / (1 + exp(-g)) */
            out[i * d + j] = sg * u;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Step 4: INT8 x INT8 -> INT32 GEMM [GEMM-IF], [SKILL], [DAY25].       */
/* ------------------------------------------------------------------ */

static int8_t weight_at(const int8_t *b, int layout, int64_t n, int64_t k, int64_t kk, int64_t j)
{
    return layout == OR_B_KN ? b[kk * n + j] : b[j * k + kk];
}

/* Returns the number of accumulators that do not fit in int32 (0 = all fit). */
int64_t or_gemm_i32(int64_t m, int64_t n, int64_t k, const int8_t *a, const int8_t *b,
                    int layout, int32_t *c)
{
    int64_t overflow = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : overflow)
    for (int64_t i = 0; i < m; ++i) {
        int64_t *acc = (int64_t *)calloc((size_t)(n > 0 ? n : 1), sizeof(int64_t));
        if (layout == OR_B_KN) {
            for (int64_t kk = 0; kk < k; ++kk) {
                int64_t av = a[i * k + kk];
                for (int64_t j = 0; j < n; ++j)
                    acc[j] += av * (int64_t)b[kk * n + j];
            }
        } else {
            for (int64_t j = 0; j < n; ++j)
                for (int64_t kk = 0; kk < k; ++kk)
                    acc[j] += (int64_t)a[i * k + kk] * (int64_t)b[j * k + kk];
        }
        for (int64_t j = 0; j < n; ++j) {
            if (acc[j] > INT32_MAX || acc[j] < INT32_MIN)
                ++overflow;
            c[i * n + j] = (int32_t)acc[j];
        }
        free(acc);
    }
    return overflow;
}

/* Accumulators for the listed (row, col) pairs only, one dot product each. */
int64_t or_gemm_entries(int64_t count, const int64_t *rows, const int64_t *cols, int64_t n,
                        int64_t k, const int8_t *a, const int8_t *b, int layout, int32_t *c)
{
    int64_t overflow = 0;
#pragma omp parallel for schedule(static) reduction(+ : overflow)
    for (int64_t e = 0; e < count; ++e) {
        int64_t acc = 0;
        for (int64_t kk = 0; kk < k; ++kk)
            acc += (int64_t)a[rows[e] * k + kk] * (int64_t)weight_at(b, layout, n, k, kk, cols[e]);
        if (acc > INT32_MAX || acc < INT32_MIN)
            ++overflow;
        c[e] = (int32_t)acc;
    }
    return overflow;
}

/* ------------------------------------------------------------------ */
/* Step 5: dequant epilogue [GEMM-IF], [DAY25], in binary64.            */
/* ------------------------------------------------------------------ */

/* out[i][j] = acc[i][j] * scale_a[i] * scale_b[j] * output_scale */
void or_dequant(int64_t m, int64_t n, const int32_t *c, const float *scale_a,
                const float *scale_b, float output_scale, double *out)
{
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            out[i * n + j] = (double)c[i * n + j] * (double)scale_a[i] * (double)scale_b[j] *
                             (double)output_scale;
}

/* The same product for listed entries: out[e] = acc[e] * sa[e] * sb[e] * output_scale. */
void or_dequant_entries(int64_t count, const int32_t *c, const float *scale_a,
                        const float *scale_b, float output_scale, double *out)
{
    for (int64_t e = 0; e < count; ++e)
        out[e] = (double)c[e] * (double)scale_a[e] * (double)scale_b[e] * (double)output_scale;
}

/* bfloat16 (8 significant bits, binary32 exponent range) nearest v, ties to even. */
static uint16_t bf16_nearest(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7fc0;
    if (a == 0.0)
        return sign;
    if (isinf(v))
        return sign | 0x7f80;
    int e;
    frexp(a, &e);             /* a = f * 2^e, 0.5 <= f < 1: leading bit is 2^(e-1) */
    int lsb = (e - 1) - 7;    /* weight of the last of 8 significant bits */
    if (lsb < -133)
        lsb = -133;           /* subnormal spacing 2^-133 */
    double r = ldexp(nearbyint(ldexp(a, -lsb)), lsb); /* exact scalings around one RNE */
    if (r >= 0x1p128)
        return sign | 0x7f80;
    float f = (float)r;       /* exact: at most 8 significant bits, in range */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

void or_bf16_nearest(int64_t count, const double *v, uint16_t *out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = bf16_nearest(v[i]);
}

/* ------------------------------------------------------------------ */
/* FP8 path [PR]: dynamic per-token quantization to float8_e4m3fn and   */
/* the FP8 x FP8 GEMM it feeds.                                        */
/* ------------------------------------------------------------------ */

/* float8_e4m3fn (OCP): sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, S.1111.111 is NaN, the largest finite magnitude is
 * S.1111.110 = 1.75 * 2^8 = 448 (the page's fp8_max), subnormals are
 * M * 2^-9. */
double or_fp8_decode(uint8_t c)
{
    const int sign = c >> 7;
    const int e = (c >> 3) & 15;
    const int m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    /* normal: (1 + m/8) 2^(e-7) = (8 + m) 2^(e-10); subnormal: m 2^-9 */
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return sign ? -v : v;
}

/* Round to nearest, ties to even, saturating at +-448; the sign of zero is
 * kept; NaN -> S.1111.111.  All arithmetic below is exact in binary64. */
uint8_t or_fp8_encode(float v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return sign | 0x7F;
    const double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < 0x1p-6) {
        /* subnormal range: the nearest multiple of 2^-9 (8 * 2^-9 is the
         * smallest normal, whose code is 0x08) */
        const double m = nearbyint(a * 512.0);
        return sign | (uint8_t)m;
    }
    int e;
    const double f = frexp(a, &e); /* a = f 2^e, f in [0.5, 1) */
    e -= 1;                         /* a = (2f) 2^e, 2f in [1, 2) */
    double q = nearbyint((2.0 * f - 1.0) * 8.0);
    if (q == 8.0) {
        q = 0.0;
        e += 1;
    }
    if (e > 8 || (e == 8 && q == 7.0))
        return sign | 0x7E; /* rounds past 448: saturate */
    return sign | (uint8_t)(((e + 7) << 3) | (int)q);
}

void or_fp8_encode_array(int64_t count, const float *v, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = or_fp8_encode(v[i]);
}

void or_fp8_decode_array(int64_t count, const uint8_t *c, double *out)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = or_fp8_decode(c[i]);
}

/* x: [m][k] binary32 -> q: [m][k] e4m3fn codes, scale: [m].
 * scale = max(absmax, 1e-12) / 448, clamped to scale_ub when scale_ub > 0
 * [PR: "optionally clamped by scale_ub"]; code = e4m3fn(x / scale) with the
 * binary32 quotient (the same reading as the INT8 path: a true division). */
void or_quant_rows_fp8(int64_t m, int64_t k, const float *x, float scale_ub, uint8_t *q,
                       float *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        const float *row = x + i * k;
        float amax = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            float a = fabsf(row[j]);
            if (a > amax)
                amax = a;
        }
        float s = fmaxf(amax, 1e-12f) / 448.0f;
        if (scale_ub > 0.0f && s > scale_ub)
            s = scale_ub;
        scale[i] = s;
        for (int64_t j = 0; j < k; ++j) {
            float ratio = row[j] / s;
            q[i * k + j] = or_fp8_encode(ratio);
        }
    }
}

/* acc[i][j] = sum_t value(a[i][t]) * value(B(t, j)) in binary64.  Exact for
 * k <= 2^17: every product is a multiple of 2^-18 below 2^18 (448^2), so any
 * partial sum needs at most 18 + 18 + 17 = 53 significant bits. */
void or_gemm_fp8(int64_t m, int64_t n, int64_t k, const uint8_t *a, const uint8_t *b, int layout,
                 double *acc)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = or_fp8_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        double *row = acc + i * n;
        for (int64_t j = 0; j < n; ++j)
            row[j] = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            const double av = lut[a[i * k + kk]];
            for (int64_t j = 0; j < n; ++j) {
                const uint8_t bc = layout == OR_B_KN ? b[kk * n + j] : b[j * k + kk];
                row[j] += av * lut[bc];
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Per-group weight scales [DAY25-G]                                   */
/* ------------------------------------------------------------------ */

/* acc[i][j] = sum over groups g of scale_b[g][j] * P_g[i][j], where
 * P_g[i][j] = sum of a[i][t] * B(t, j) over t in [g * group, (g + 1) * group)
 * (the last group ends at k), an exact integer; scale_b is [ceil(k / group)][n].
 * Each product P_g * scale is exact in binary64 (|P_g| < 2^31, a binary32
 * scale has 24 significant bits); the sum over groups is binary64. */
void or_gemm_i8_grouped(int64_t m, int64_t n, int64_t k, int64_t group, const int8_t *a,
                        const int8_t *b, int layout, const float *scale_b, double *acc)
{
    const int64_t groups = (k + group - 1) / group;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double sum = 0.0;
            for (int64_t g = 0; g < groups; ++g) {
                int64_t partial = 0;
                const int64_t end = (g + 1) * group < k ? (g + 1) * group : k;
                for (int64_t kk = g * group; kk < end; ++kk)
                    partial += (int64_t)a[i * k + kk] * (int64_t)weight_at(b, layout, n, k, kk, j);
                sum += (double)partial * (double)scale_b[g * n + j];
            }
            acc[i * n + j] = sum;
        }
    }
}

/* out[i][j] = acc[i][j] * scale_a[i] * output_scale in binary64 */
void or_dequant_grouped(int64_t m, int64_t n, const double *acc, const float *scale_a,
                        float output_scale, double *out)
{
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            out[i * n + j] = acc[i * n + j] * (double)scale_a[i] * (double)output_scale;
}

/* ------------------------------------------------------------------ */
/* Static per-tensor scale [PR-S]                                      */
/* ------------------------------------------------------------------ */

/* code = clamp(rint(x / scale), -127, 127), one scale for every element */
void or_quant_static(int64_t count, const float *x, float scale, int8_t *q)
{
    for (int64_t i = 0; i < count; ++i) {
        float r = nearbyintf(x[i] / scale);
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        q[i] = (int8_t)r;
    }
}

/* code = e4m3fn(x / scale) */
void or_quant_static_fp8(int64_t count, const float *x, float scale, uint8_t *q)
{
    for (int64_t i = 0; i < count; ++i)
        q[i] = or_fp8_encode(x[i] / scale);
}

/* ------------------------------------------------------------------ */
/* Asymmetric per-token quantization [ASYM]                            */
/* ------------------------------------------------------------------ */

/* lo = min(row min, 0), hi = max(row max, 0);
 * scale = max(hi - lo, 1e-12) / 255                (binary32 operations);
 * zp = clamp(rint(-lo / scale) - 128, -128, 127);
 * code = clamp(rint(x / scale) + zp, -128, 127), so x ~ (code - zp) * scale
 * and x = 0 has the exact code zp. */
void or_quant_rows_asym(int64_t m, int64_t k, const float *x, int8_t *q, float *scale,
                        int32_t *zp)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        const float *row = x + i * k;
        float lo = 0.0f, hi = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            if (row[j] < lo)
                lo = row[j];
            if (row[j] > hi)
                hi = row[j];
        }
        const float s = fmaxf(hi - lo, 1e-12f) / 255.0f;
        float z = nearbyintf(-lo / s) - 128.0f;
        if (z > 127.0f)
            z = 127.0f;
        if (z < -128.0f)
            z = -128.0f;
        scale[i] = s;
        zp[i] = (int32_t)z;
        for (int64_t j = 0; j < k; ++j) {
            float r = nearbyintf(row[j] / s) + z;
            if (r > 127.0f)
                r = 127.0f;
            if (r < -128.0f)
                r = -128.0f;
            q[i * k + j] = (int8_t)r;
        }
    }
}

/* acc[i][j] = sum_t (a[i][t] - zp[i]) * B(t, j), exact; returns the number of
 * results outside int32. */
int64_t or_gemm_asym(int64_t m, int64_t n, int64_t k, const int8_t *a, const int32_t *zp,
                     const int8_t *b, int layout, int32_t *c)
{
    int64_t overflow = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : overflow)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            int64_t acc = 0;
            for (int64_t kk = 0; kk < k; ++kk)
                acc += ((int64_t)a[i * k + kk] - zp[i]) * (int64_t)weight_at(b, layout, n, k, kk, j);
            if (acc > INT32_MAX || acc < INT32_MIN)
                ++overflow;
            c[i * n + j] = (int32_t)acc;
        }
    }
    return overflow;
}
