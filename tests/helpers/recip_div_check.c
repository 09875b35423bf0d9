/* Checks, in IEEE binary32 with fused multiply-add, the quotient the library's encode computes for
 * the block scale: RN(a / b) as q0 = RN(a y) with y = RN(1 / b), then two residual corrections
 * q <- RN(q + RN(a - q b) y) (fmaf).  Prints "checked bad" for each of three samples:
 *   1. b = 6 and every a in [2^lo, 2^hi) (argv 1, 2: exponents), stride argv 3;
 *   2. argv 4 random b in [2^-100, 2^100], 2 * 10^5 random a each, half of them next to b times a
 *      short number (quotients near short values and rounding midpoints);
 *   3. the scale byte: E4M3 rounding of min(RN(RN(ab / T) / ts), 448) from the two corrected
 *      quotients against IEEE division, for the targets T = 6, 5.5, 5, 4.5 and 4 in turn, argv 5
 *      random ts with 10^5 block maxima each, from 2^-40 to 2^12 times the tensor maximum 2688 ts
 *      (quotients down into the subnormal range). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float corrected_quotient(float a, float b, float y) {
  volatile float q = a * y; /* a separate multiply, not contracted into the fma below */
  float r = fmaf(-q, b, a);
  float q1 = fmaf(r, y, q);
  r = fmaf(-q1, b, a);
  return fmaf(r, y, q1);
}

static uint32_t e4m3_byte(float s) { /* E4M3 round-to-nearest-even of 0 <= s <= 448 */
  if (s < 0.015625f) {
    volatile float t = s * 512.0f;
    return (uint32_t)rintf(t);
  }
  uint32_t b = f2u(s);
  uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
  return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
}

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
  st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
  return (uint32_t)((st * 0x2545F4914F6CDD1Dull) >> 32);
}

int main(int argc, char **argv) {
  if (argc < 6) return 2;
  const int lo = atoi(argv[1]), hi = atoi(argv[2]);
  const uint32_t stride = (uint32_t)atoi(argv[3]);
  const int nb = atoi(argv[4]), nts = atoi(argv[5]);
  volatile float one = 1.0f, six = 6.0f;
  long n = 0, bad = 0;
  const float y6 = one / six;
  for (uint32_t u = f2u(ldexpf(1.0f, lo)); u < f2u(ldexpf(1.0f, hi)); u += stride) {
    const float a = u2f(u);
    volatile float ref = a / six;
    ++n;
    if (f2u(corrected_quotient(a, 6.0f, y6)) != f2u(ref)) ++bad;
  }
  printf("%ld %ld\n", n, bad);
  n = bad = 0;
  for (int ib = 0; ib < nb; ++ib) {
    const float b = u2f(((uint32_t)(127 - 100 + rnd() % 201) << 23) | (rnd() & 0x7FFFFF));
    const float y = one / b;
    for (int ia = 0; ia < 200000; ++ia) {
      float a = u2f(((uint32_t)(127 - 93 + rnd() % 217) << 23) | (rnd() & 0x7FFFFF));
      if (ia & 1) {
        const float k = (float)(1 + rnd() % 1000) * u2f((uint32_t)(127 - 10 + rnd() % 20) << 23);
        volatile float t = b * k;
        a = u2f(f2u(t) + (uint32_t)(rnd() % 5) - 2u);
        if (!(a >= 0x1p-93f && a <= 0x1p124f)) continue;
      }
      volatile float ref = a / b;
      if (!(ref >= 0x1p-126f) || isinf(ref)) continue;
      ++n;
      if (f2u(corrected_quotient(a, b, y)) != f2u(ref)) ++bad;
    }
  }
  printf("%ld %ld\n", n, bad);
  n = bad = 0;
  static const float targets[5] = {6.0f, 5.5f, 5.0f, 4.5f, 4.0f};
  for (int it = 0; it < nts; ++it) {
    volatile float T = targets[it % 5];
    const float yT = one / T;
    const float ts = u2f(((uint32_t)(127 - 100 + rnd() % 201) << 23) | (rnd() & 0x7FFFFF));
    const float yts = one / ts;
    volatile float amax = ts * 2688.0f;
    for (int ia = 0; ia < 100000; ++ia) {
      const float ab = ldexpf(amax, (int)(rnd() % 53) - 40) * u2f(0x3f800000u | (rnd() & 0x7FFFFF)) * 0.75f;
      if (!(ab >= 0x1p-90f && ab <= 0x1p100f)) continue;
      volatile float q = ab / T;
      volatile float s = q / ts;
      const float sf = fminf(corrected_quotient(corrected_quotient(ab, T, yT), ts, yts), 448.0f);
      ++n;
      if (e4m3_byte(fminf(s, 448.0f)) != e4m3_byte(sf)) ++bad;
    }
  }
  printf("%ld %ld\n", n, bad);
  return 0;
}
