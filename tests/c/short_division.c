/* Check, for every finite positive binary16 divisor d (normal and subnormal)
 * and many binary32 dividends a, the quotient
 *     q0 = RN(a * y), r = RN(fma(-q0, d, a)), q = RN(fma(r, y, q0)),  y = RN(1/d)
 * against the correctly rounded RN(a / d).  The quantizers divide by an FP16
 * step or scale this way and keep rint(q).  Prints: mismatches, cases,
 * mismatches with a and a/d both normal, mismatches that change rint(q). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f16_to_f32(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  if (e == 0) return ldexpf((float)m, -24);
  return ldexpf((float)(m | 1024), e - 25);
}

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next(void) { /* xorshift64* */
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}

static long bad_normal = 0, bad_code = 0;

static int check(float a, float d, float y) {
  const float q0 = a * y;
  const float r = fmaf(-q0, d, a);
  const float q = fmaf(r, y, q0);
  const float want = a / d;
  if (memcmp(&q, &want, 4) == 0) return 0;
  if (fabsf(a) >= 0x1p-126f && fabsf(want) >= 0x1p-126f) ++bad_normal;
  if (rintf(q) != rintf(want)) ++bad_code;
  return 1;
}

int main(int argc, char **argv) {
  int per_divisor = argc > 1 ? atoi(argv[1]) : 2000;
  long bad = 0, n = 0;
  for (uint32_t h = 1; h < 0x7C00; ++h) {
    const float d = f16_to_f32((uint16_t)h);
    const float y = 1.0f / d;
    /* dividends: small integers times d (exact quotients), their neighbours,
       and random binary32 values over the range a quantizer sees */
    for (int k = -40; k <= 40; ++k) {
      const float a = (float)k * d;
      bad += check(a, d, y) + check(nextafterf(a, INFINITY), d, y) + check(nextafterf(a, -INFINITY), d, y);
      n += 3;
    }
    for (int i = 0; i < per_divisor; ++i) {
      uint32_t bits = next();
      const uint32_t e = 127 + ((int)(next() % 40) - 20); /* |a| within 2^-20 .. 2^20 of 1 */
      bits = (bits & 0x807FFFFFu) | (e << 23);
      float a;
      memcpy(&a, &bits, 4);
      a *= d; /* keep a/d in the range the quantizers use */
      bad += check(a, d, y);
      ++n;
    }
  }
  printf("%ld %ld %ld %ld\n", bad, n, bad_normal, bad_code);
  return 0;
}
