/* The store's binary32 quotient without a division per element (see
 * Divisor / quotient in csrc/store_row.h), restated in C with C99 fmaf:
 * r = RN(1/s), q0 = RN(x r), q1 = RN(q0 + RN(x - s q0) r). Checked against
 * the IEEE quotient RN(x/s) for every finite BF16 x and `nscale` scales in
 * [2^-60, 2^60] (powers of two, amax/448 around 1, random). Where the store
 * keeps q0 (|x| or |q0| below 2^-100, |q0| above 2^100), q0 must have the
 * quotient's sign and both must lie below 2^-40 (a signed-zero code) or
 * above 2^99 (a saturated code). Prints the counts; exit status 1 on any
 * failure. Usage: quotient_check NSCALE */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits2f(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t f2bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
static uint64_t rng = 88172645463325252ull;
static uint32_t xr(void) { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return (uint32_t)rng; }

int main(int argc, char** argv) {
  const int nscale = argc > 1 ? atoi(argv[1]) : 2000;
  long exact = 0, kept = 0, bad = 0;
  for (int si = 0; si < nscale; ++si) {
    float s;
    if (si < 121) s = ldexpf(1.0f, si - 60);
    else if (si < 121 + nscale / 4) s = bits2f(0x3f800000u + (uint32_t)(si * 997u % 0x800000u)) / 448.0f;
    else s = bits2f(((uint32_t)(127 - 60 + xr() % 121) << 23) | (xr() & 0x7fffff));
    if (!(s >= 0x1p-60f && s <= 0x1p60f)) continue;
    volatile float one = 1.0f, sv = s;
    const float r = one / sv;
    for (uint32_t xb = 0; xb < 65536; ++xb) {
      const float x = bits2f(xb << 16);
      if (!isfinite(x)) continue;
      volatile float xv = x;
      const float qref = xv / sv;
      const float q0 = x * r;
      const float aq = fabsf(q0);
      if (fabsf(x) >= 0x1p-100f && aq >= 0x1p-100f && aq <= 0x1p100f) {
        const float q1 = fmaf(fmaf(-s, q0, x), r, q0);
        ++exact;
        if (f2bits(q1) != f2bits(qref)) {
          if (bad < 5) printf("quotient differs: x=%a s=%a ieee=%a got=%a\n", x, s, qref, q1);
          ++bad;
        }
      } else {
        ++kept;
        const int same_sign = (signbit(q0) != 0) == (signbit(qref) != 0);
        const int tiny = aq < 0x1p-40f && fabsf(qref) < 0x1p-40f;
        const int huge = aq >= 0x1p100f && fabsf(qref) >= 0x1p99f;
        if (!same_sign || !(tiny || huge)) {
          if (bad < 5) printf("kept q0 differs in code: x=%a s=%a ieee=%a q0=%a\n", x, s, qref, q0);
          ++bad;
        }
      }
    }
  }
  printf("exact %ld kept %ld bad %ld\n", exact, kept, bad);
  return bad != 0;
}
