/*
 * Host check of the requantiser's quotient (fp8_gemv_amd/csrc/requant.hip): for a block scale
 * d = RN(amax / 127) the kernel forms each v / d as
 *     k = 2^64 if d < 2^-60, 2^-64 if d > 2^60, else 1;  ds = d * k;  rcp = RN(1 / ds)
 *     q0 = RN(v * k * rcp);  q = fma(fma(-q0, ds, v * k), rcp, q0)
 * and relies on q being the IEEE quotient RN(v / d).  Here that is checked for every pair of
 * e4m3 codes (block maximum, element with |v| <= amax) at each of N scales S, with
 * v = RN(e4m3 * S): powers of two, 1, 0.3, and random floats from the subnormals to 2^118.
 * Equality is by value and by the rounded integer (a -0 quotient may come back +0).
 * Prints the number of checks and mismatches; exit status 1 on any mismatch.
 * Compile with -ffp-contract=off (no contraction other than the explicit fmaf).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float e4m3(int c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  const float v = e == 0 ? ldexpf((float)m / 8.0f, -6) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return s ? -v : v;
}

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}

int main(int argc, char **argv) {
  const int nscales = argc > 1 ? atoi(argv[1]) : 2000;
  long checks = 0, bad = 0;
  for (int si = 0; si < nscales; ++si) {
    float S;
    if (si == 0) S = 1.0f;
    else if (si == 1) S = 0.3f;
    else if (si < 48) S = ldexpf(1.0f, -140 + 6 * si);
    else {
      uint32_t bits = (uint32_t)(next() >> 32) & 0x007FFFFFu;
      bits |= (uint32_t)(next() % 246) << 23;  /* exponent field 0 (subnormal) .. 245 */
      memcpy(&S, &bits, 4);
    }
    for (int ca = 1; ca < 127; ++ca) {
      const float amax = fabsf(e4m3(ca) * S);
      const float d = amax / 127.0f;
      if (!(d > 0.0f) || !isfinite(amax)) continue;
      const float k = d < 0x1p-60f ? 0x1p64f : (d > 0x1p60f ? 0x1p-64f : 1.0f);
      const float ds = d * k;
      const float rcp = 1.0f / ds;
      for (int c = 0; c < 256; ++c) {
        if ((c & 0x7F) == 0x7F) continue; /* NaN codes */
        const float v = e4m3(c) * S;
        if (fabsf(v) > amax) continue;
        const float ref = v / d;
        const float vs = v * k;
        const float q0 = vs * rcp;
        const float q = fmaf(fmaf(-q0, ds, vs), rcp, q0);
        ++checks;
        if (!(q == ref) || (int)roundf(q) != (int)roundf(ref)) {
          if (++bad <= 5) printf("S=%a v=%a d=%a ieee=%a kernel=%a\n", S, v, d, ref, q);
        }
      }
    }
  }
  printf("checks %ld mismatches %ld\n", checks, bad);
  return bad != 0;
}
