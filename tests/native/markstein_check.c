/* Checks, on the CPU in IEEE fp32 with correctly rounded fma, the identities
 * the Q8_1 block rule of the kernels relies on to reach correctly rounded
 * quotients without a division instruction (Markstein's theorem: with y the
 * correctly rounded reciprocal of b and q0 = RN(a*y), the residual a - q0*b is
 * exact in one fma and RN(q0 + residual*y) = RN(a/b)).
 *   mode 1: d = fma(fma(-q0, 127, a), RN(1/127), q0), q0 = a*RN(1/127), equals
 *           a/127 for every float a in the binades [2^e0, 2^e1) and every
 *           denormal.
 *   mode 2: one Newton step y1 = fma(fma(-d, y0, 1), y0, y0) from either float
 *           within one ulp of 1/d gives RN(1/d), for every significand of d but
 *           one: from the lower neighbour of the all-ones significand
 *           (d = 2 - 2^-23, y0 = 1/2), Markstein's exception, which mode 2
 *           counts apart and prints as a fourth field.
 *   mode 3: q1 = fma(fma(-q0, d, x), y, q0), q0 = x*y, y = RN(1/d), equals x/d
 *           for n_div divisors (extremes and seeded significands) and every x
 *           in [1, 4).
 * Prints one line "<mode> <tested> <mismatches>"; exit status 0 when none. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static long check_d(uint32_t lo, uint32_t hi, long* tested) {
  const float y = 1.0f / 127.0f;
  long bad = 0;
  for (uint32_t u = lo; u < hi; ++u) {
    const float a = f_of(u);
    const float q0 = a * y;
    const float d = fmaf(fmaf(-q0, 127.0f, a), y, q0);
    bad += u_of(d) != u_of(a / 127.0f);
    ++*tested;
  }
  return bad;
}

int main(int argc, char** argv) {
  const int mode = argc > 1 ? atoi(argv[1]) : 0;
  long tested = 0, bad = 0, exception = 0;
  if (mode == 1) {
    const int e0 = atoi(argv[2]), e1 = atoi(argv[3]);
    bad += check_d(0u, 0x00800000u, &tested);                      /* denormals */
    bad += check_d((uint32_t)(e0 + 127) << 23, (uint32_t)(e1 + 127) << 23, &tested);
  } else if (mode == 2) {
    for (uint32_t m = 0; m < (1u << 23); ++m) {
      const float d = f_of(0x3f800000u | m);
      const float t = 1.0f / d;
      const double ex = 1.0 / (double)d;
      for (int k = -1; k <= 1; ++k) {
        const float y0 = f_of(u_of(t) + k);
        int e;
        frexp(ex, &e);                       /* ex in [2^(e-1), 2^e): its ulp is 2^(e-24) */
        if (fabs((double)y0 - ex) >= ldexp(1.0, e - 24)) continue;   /* starts within one ulp */
        const float y1 = fmaf(fmaf(-d, y0, 1.0f), y0, y0);
        if (u_of(y1) != u_of(t)) {
          if (m == 0x7fffffu && k == -1) ++exception; else ++bad;
        }
        ++tested;
      }
    }
  } else if (mode == 3) {
    const int n_div = atoi(argv[2]);
    uint64_t s = 0x9e3779b97f4a7c15ull;
    for (int i = 0; i < n_div; ++i) {
      uint32_t md;
      if (i == 0) md = 0; else if (i == 1) md = 0x7fffff; else if (i == 2) md = 1;
      else { s = s * 6364136223846793005ull + 1442695040888963407ull; md = (uint32_t)(s >> 41); }
      const float d = f_of(0x3f800000u | md);
      const float y = 1.0f / d;
      for (uint32_t u = 0x3f800000u; u < 0x40800000u; ++u) {
        const float x = f_of(u);
        const float q0 = x * y;
        const float q1 = fmaf(fmaf(-q0, d, x), y, q0);
        bad += u_of(q1) != u_of(x / d);
        ++tested;
      }
    }
  } else {
    fprintf(stderr, "usage: markstein_check 1 e0 e1 | 2 | 3 n_div\n");
    return 2;
  }
  if (mode == 2)
    printf("%d %ld %ld %ld\n", mode, tested, bad, exception);
  else
    printf("%d %ld %ld\n", mode, tested, bad);
  return bad ? 1 : 0;
}
