/* Host-side check of the division the accumulation's exact pass uses in float64: for a divisor b,
 * y = RN(1/b) once, then per dividend m
 *     q = RN(m y),  r = m - b q (exact, one FMA),  result = RN(q + r y)  (one FMA),
 * which Markstein's theorem makes equal to RN(m / b) whenever y = RN(1/b) and q is within an ulp
 * of m / b, barring underflow and overflow.  The cases have the exact pass's shape: m = s h with
 * s a float32 scale in [2^-60, 2^61) and h a multiple of 2^-9 below 2^18 (the exact transform of
 * decoded codes), b a float32 alpha in [2^-126, 2^127) or the float64 sqrt(128), sqrt(512).
 * Prints "ok <cases>" or the first mismatches.  Built with contraction off, so that m y and the
 * FMAs are exactly the operations named. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) { /* xorshift64 */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
static float random_float(int emin, int emax) { /* positive normal float32, exponent in [emin, emax] */
  const uint32_t mant = (uint32_t)(next() & 0x7FFFFF);
  const int e = emin + (int)(next() % (uint64_t)(emax - emin + 1));
  const uint32_t bits = ((uint32_t)(e + 127) << 23) | mant;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

int main(int argc, char **argv) {
  const long cases = argc > 1 ? atol(argv[1]) : 20000000L;
  const double roots[2] = {sqrt(128.0), sqrt(512.0)};
  long bad = 0, n = 0;
  for (long i = 0; i < cases; ++i) {
    const float s = random_float(-60, 60), a = random_float(-126, 126);
    const double h = (double)((int64_t)(next() % 268435457ull) - 134217728) * 0x1p-9;
    const double m = (double)s * h; /* exact: 24 + 27 bits */
    const double b = (i & 1) ? (double)a : roots[(i >> 1) & 1];
    const double y = 1.0 / b;
    const double q = m * y;
    const double got = fma(fma(-q, b, m), y, q);
    const double want = m / b;
    ++n;
    if (got != want && !(got == 0.0 && want == 0.0)) {
      if (bad < 5) printf("m=%a b=%a want=%a got=%a\n", m, b, want, got);
      ++bad;
    }
  }
  if (bad) {
    printf("%ld of %ld differ\n", bad, n);
    return 1;
  }
  printf("ok %ld\n", n);
  return 0;
}
