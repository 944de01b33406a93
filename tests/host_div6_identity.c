/* Host check of an arithmetic identity the device quantizer relies on:
 * for every binary32 x in [2^-125, FLT_MAX],
 *     q = x * RN(1/6);  e = fma(-q, 6, x);  q = fma(e, RN(1/6), q)
 * equals the correctly rounded quotient x / 6.  IEEE binary32 multiply and
 * fma round identically on the host and on gfx950 (denormals kept), so the
 * check carries over.  Prints the number of mismatches (expected 0). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

int main(void) {
  const float r = 1.0f / 6.0f;
  unsigned long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (long long b = 0x01000000LL; b <= 0x7F7FFFFFLL; ++b) {
    const uint32_t u = (uint32_t)b;
    float x;
    memcpy(&x, &u, 4);
    volatile float want = x / 6.0f;
    float q = x * r;
    const float e = fmaf(-q, 6.0f, x);
    q = fmaf(e, r, q);
    if (q != want) ++bad;
  }
  printf("%llu\n", bad);
  return 0;
}
