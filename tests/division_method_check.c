/* Checks, on the CPU, the division method of the GPU quantization kernel:
 * with s = max(amax, 1e-12f) / 127 and r = 1 / s (both correctly rounded),
 *   y = x * r;  e = fma(-y, s, x);  q = fma(e, r, y)
 * must give the same integer code clamp(rint(.), -127, 127) as the IEEE
 * quotient x / s, and the same quotient whenever |x / s| >= 2^-20.
 * Exhaustive over bf16 inputs for a set of bf16 row maxima, plus random
 * binary32 inputs (a share of them placed next to half-integer multiples
 * of s, where a wrong quotient would change the code).  Prints mismatches.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static float clampi(float q) { q = rintf(q); return q > 127.f ? 127.f : (q < -127.f ? -127.f : q); }

static uint64_t st = 0x9e3779b97f4a7c15ull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }

static long long bad = 0;
static void check(float x, float s, float r) {
  float q1 = x / s;
  float y = x * r;
  float e = fmaf(-y, s, x);
  float q2 = fmaf(e, r, y);
  if (clampi(q1) != clampi(q2) || (fabsf(q1) >= 0x1p-20f && q1 != q2)) {
    if (bad < 5) printf("mismatch x=%a s=%a ieee=%a method=%a\n", x, s, q1, q2);
    ++bad;
  }
}

int main(int argc, char **argv) {
  long long nrand = argc > 1 ? atoll(argv[1]) : 20000000LL;
  long long total = 0;
  for (uint32_t ab = 0x0080; ab < 0x7f80; ab += 97) { /* bf16 row maxima */
    float amax = from_bits(ab << 16);
    float s = fmaxf(amax, 1e-12f) / 127.0f, r = 1.0f / s;
    for (uint32_t xb = 0; xb < 0x7f80; ++xb) {
      float x = from_bits(xb << 16);
      if (x > amax) break;
      check(x, s, r); check(-x, s, r); total += 2;
    }
  }
  for (long long i = 0; i < nrand; ++i) {
    float amax = fabsf(from_bits((uint32_t)rnd()));
    if (!isfinite(amax)) continue;
    float s = fmaxf(amax, 1e-12f) / 127.0f, r = 1.0f / s;
    uint64_t u = rnd();
    float x = ((u >> 40) & 1 ? -1.f : 1.f) * (from_bits(((uint32_t)u & 0x7fffff) | 0x3f800000) - 1.f) * amax;
    if ((i & 3) == 0) {
      int j = (int)(rnd() % 254) - 127;
      x = nextafterf((j + 0.5f) * s, (rnd() & 1) ? INFINITY : -INFINITY);
      if (fabsf(x) > amax) continue;
    }
    check(x, s, r); ++total;
  }
  printf("checked %lld mismatches %lld\n", total, bad);
  return bad != 0;
}
