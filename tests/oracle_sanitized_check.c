/* Runs the CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (host code only; test infrastructure): quantization of random and edge
 * rows, the silu product, the GEMM at the INT32 closed forms K = 65536
 * (|q| = 127) and K = 131056 (-128 * -128, the largest K accepted), the
 * dequant and the bf16 rounding.  Any out-of-bounds access, signed overflow
 * or other undefined behaviour aborts with a report; the closed forms are
 * checked as well. */
#include "../oracle/qk_oracle.c"

#include <stdio.h>
#include <stdlib.h>

static uint32_t lcg(uint32_t *st) { *st = *st * 1664525u + 1013904223u; return *st; }

static int gemm_closed_form(int64_t k, int8_t av, int8_t bv)
{
    const int64_t m = 2, n = 64;
    int8_t *a = malloc((size_t)(m * k));
    int8_t *b = malloc((size_t)(k * n));
    int32_t *c = malloc(sizeof(int32_t) * (size_t)(m * n));
    if (!a || !b || !c) return 1;
    memset(a, av, (size_t)(m * k));
    memset(b, bv, (size_t)(k * n));
    const int64_t out_of_range = or_gemm_i32(m, n, k, a, b, OR_B_KN, c);
    int bad = out_of_range != 0;
    for (int64_t i = 0; i < m * n; ++i)
        bad |= (int64_t)c[i] != k * av * bv;
    free(a); free(b); free(c);
    if (bad) printf("closed form K=%lld a=%d b=%d failed\n", (long long)k, av, bv);
    return bad;
}

int main(void)
{
    uint32_t st = 12345u;
    /* quantization: random rows, a zero row, rows of extremes and subnormals */
    enum { M = 9, K = 1000 };
    float *x = malloc(sizeof(float) * M * K);
    int8_t *q = malloc(M * K);
    float *s = malloc(sizeof(float) * M);
    if (!x || !q || !s) return 1;
    for (int i = 0; i < M * K; ++i) x[i] = ((float)(lcg(&st) >> 8) / 16777216.0f - 0.5f) * 8.0f;
    for (int j = 0; j < K; ++j) x[1 * K + j] = 0.0f;
    for (int j = 0; j < K; ++j) x[2 * K + j] = (j & 1) ? 3.4e38f : -3.4e38f;
    for (int j = 0; j < K; ++j) x[3 * K + j] = (float)j * 1e-41f;
    or_quant_rows(M, K, x, q, s);
    for (int i = 0; i < M * K; ++i)
        if (q[i] < -127) { printf("code -128\n"); return 1; }

    /* silu(gate) * up over a spread of gates */
    enum { D = 512 };
    float *h = malloc(sizeof(float) * 2 * D), *y = malloc(sizeof(float) * D);
    if (!h || !y) return 1;
    for (int j = 0; j < 2 * D; ++j) h[j] = ((float)(lcg(&st) >> 8) / 16777216.0f - 0.5f) * 240.0f;
    or_silu_mul(1, D, h, y);

    /* GEMM closed forms at the INT32 limits */
    if (gemm_closed_form(65536, 127, 127)) return 1;
    if (gemm_closed_form(65536, 127, -127)) return 1;
    if (gemm_closed_form(131056, -128, -128)) return 1;

    /* dequant and bf16 rounding */
    int32_t cc[4] = {2147483647, -2147483647 - 1, 0, 12345};
    float sa[2] = {1e-3f, 3.0f}, sb[2] = {0.5f, 1e-2f};
    double out[4];
    or_dequant(2, 2, cc, sa, sb, 1.0f, out);
    uint16_t bf[4];
    or_bf16_nearest(4, out, bf);

    free(x); free(q); free(s); free(h); free(y);
    printf("sanitized oracle run: ok\n");
    return 0;
}
