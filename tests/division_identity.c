/*
 * division_identity.c -- host check of the quotient rule the prefill
 * epilogues use for o = acc / l.
 *
 * Claim (Markstein's correction step with a correctly rounded reciprocal,
 * P. Markstein, "IA-64 and Elementary Functions", 2000): in binary32 with
 * round-to-nearest-even, for y = RN(1/b), q0 = RN(a*y),
 * r = RN(a - q0*b) (one FMA, exact) and q1 = RN(q0 + r*y) (one FMA),
 * q1 == RN(a/b) whenever nothing underflows.  The kernels rely on it for
 * b in [1, 2^40) and |a/b| >= 2^-100 and divide otherwise.
 *
 * Checked here over every significand of b against seeded significands of a,
 * and every significand of a against seeded significands of b (plus b with
 * significand 1.0 and 1.11..1), exponents of b in [0, 40) and of a in
 * [-60, 100), both signs of a.  Prints the number of pairs and of mismatches;
 * exits non-zero on any mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t u_of(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

static int same_as_division(float a, float b) {
  const float y = 1.0f / b;
  const float q0 = a * y;
  const float r = fmaf(-q0, b, a);
  const float q1 = fmaf(r, y, q0);
  return u_of(q1) == u_of(a / b);
}

static uint64_t next(uint64_t* s) {
  *s ^= *s << 13;
  *s ^= *s >> 7;
  *s ^= *s << 17;
  return *s;
}

int main(int argc, char** argv) {
  const int per = argc > 1 ? atoi(argv[1]) : 8;
  long long total = 0, bad = 0;
#pragma omp parallel for reduction(+ : total, bad) schedule(static)
  for (uint32_t m = 0; m < (1u << 23); ++m) {
    uint64_t s = 0x9E3779B97F4A7C15ull * (m + 1);
    for (int k = 0; k < per; ++k) {
      const uint64_t x = next(&s);
      const uint32_t other = k == 0 ? 0u : k == 1 ? 0x7fffffu : (uint32_t)(x & 0x7fffff);
      const uint32_t eb = (uint32_t)((x >> 23) % 40), ea = (uint32_t)((x >> 33) % 160);
      const uint32_t sa = (uint32_t)(x >> 45) & 1u;
      /* b takes the significand m, a a seeded one ... */
      float b = f_of(((127u + eb) << 23) | m);
      float a = f_of((sa << 31) | ((127u + ea - 60u) << 23) | other);
      total++;
      if (!same_as_division(a, b)) {
        bad++;
        if (bad <= 5) printf("mismatch a=%a b=%a\n", (double)a, (double)b);
      }
      /* ... and the other way round. */
      b = f_of(((127u + eb) << 23) | other);
      a = f_of((sa << 31) | ((127u + ea - 60u) << 23) | m);
      total++;
      if (!same_as_division(a, b)) {
        bad++;
        if (bad <= 5) printf("mismatch a=%a b=%a\n", (double)a, (double)b);
      }
    }
  }
  printf("pairs %lld mismatches %lld\n", total, bad);
  return bad != 0;
}
