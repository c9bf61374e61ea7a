/* The quantization kernels form the per-token scale max(amax, 1e-12f) / d,
 * d = 127 (INT8) or 448 (FP8), as y = a * c, e = fma(-y, d, a),
 * s = fma(e, c, y) with c = RN(1/d) (Markstein's correction with a constant
 * reciprocal).  This program checks, for every binary32 value a from 1e-12f
 * (the guard) to the largest finite value, that s equals the IEEE quotient
 * a / d bit for bit; d is the first argument (default 127).  Test
 * infrastructure only: it shares nothing with the kernels but the recipe it
 * checks, written out here. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, sizeof f); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, sizeof u); return u; }

int main(int argc, char **argv) {
  const int di = argc > 1 ? atoi(argv[1]) : 127;
  const float d = (float)di;
  /* 1/d is not a binary32 midpoint for d = 127 or 448 (its binary expansion
   * does not terminate), so rounding the double quotient gives RN(1/d) */
  const float c = (float)(1.0 / (double)di);
  if (di == 127 && c != 0x1.020408p-7f) {
    printf("the constant is not RN(1/127)\n");
    return 1;
  }
  const uint32_t lo = u_of(1e-12f), hi = 0x7F7FFFFFu;
  unsigned long long n = 0, bad = 0;
  for (uint32_t u = lo;; ++u) {
    const float a = f_of(u);
    const float y = a * c;
    const float e = fmaf(-y, d, a);
    const float s = fmaf(e, c, y);
    const float ref = a / d;
    if (u_of(s) != u_of(ref)) {
      if (bad < 5) printf("mismatch at a = %a: %a vs %a\n", a, s, ref);
      ++bad;
    }
    ++n;
    if (u == hi) break;
  }
  printf("divisor %d, constant %a: checked %llu values: mismatches %llu\n", di, c, n, bad);
  return bad != 0;
}
