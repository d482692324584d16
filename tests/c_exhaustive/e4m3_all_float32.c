/*
 * e4m3_all_float32.c - the oracle's E4M3FN encoder on every one of the 2^32 float32 bit
 * patterns, against a brute-force nearest-value search written here from the format alone.
 *
 * Format (OCP 8-bit floating point, E4M3FN): sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 holds the subnormals m * 2^-9; 0x7F / 0xFF are NaN and there is no
 * infinity, so the largest finite magnitude is 0x7E = 448.  Encoding, as the oracle defines it:
 * the nearest finite value, a tie going to the code with an even mantissa, magnitudes beyond 448
 * saturating to +-448, and the sign kept (a negative value that rounds to zero is 0x80).
 *
 * The reference below tabulates the 127 non-negative finite magnitudes from the field layout,
 * finds the two that bracket |v| by bisection and picks the nearer one: no frexp, no rounding
 * primitive, nothing shared with the oracle's arithmetic.  Float32 NaN patterns are skipped
 * (outside the contract).  Prints "ok <count>" and exits 0 when every pattern agrees.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tfp8_oracle.h"

static double mag[127]; /* magnitude of code c, c = 0 .. 0x7E (increasing) */

static uint8_t reference(float f) {
  const uint8_t sign = signbit(f) ? 0x80 : 0x00;
  const double a = fabs((double)f);
  if (a >= mag[126]) return sign | 0x7E; /* 448 and beyond (infinities included) */
  int lo = 0, hi = 126;                  /* mag[lo] <= a < mag[hi] */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (mag[mid] <= a)
      lo = mid;
    else
      hi = mid;
  }
  const double below = a - mag[lo], above = mag[hi] - a;
  int c;
  if (below < above)
    c = lo;
  else if (above < below)
    c = hi;
  else
    c = (lo & 1) ? hi : lo; /* tie: the even mantissa (the code's lowest bit) */
  return sign | (uint8_t)c;
}

int main(void) {
  for (int c = 0; c < 127; ++c) {
    const int e = c >> 3, m = c & 7;
    mag[c] = e == 0 ? m * (1.0 / 512.0) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  }
  long long mismatches = 0, checked = 0;
  long long first = -1;
#pragma omp parallel for schedule(static) reduction(+ : mismatches, checked)
  for (long long u = 0; u < (1LL << 32); ++u) {
    const uint32_t bits = (uint32_t)u;
    float f;
    memcpy(&f, &bits, sizeof f);
    if (isnan(f)) continue;
    ++checked;
    if (tfp8_ref_e4m3_encode((double)f) != reference(f)) {
      ++mismatches;
#pragma omp critical
      if (first < 0 || u < first) first = u;
    }
  }
  if (mismatches) {
    uint32_t b = (uint32_t)first;
    float f;
    memcpy(&f, &b, sizeof f);
    printf("FAIL %lld of %lld patterns differ; first 0x%08x (%.9g): oracle 0x%02x, reference "
           "0x%02x\n",
           mismatches, checked, b, f, tfp8_ref_e4m3_encode((double)f), reference(f));
    return 1;
  }
  printf("ok %lld\n", checked);
  return 0;
}
