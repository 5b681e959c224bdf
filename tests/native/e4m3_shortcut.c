/* Host check of the quantiser's division shortcut: for an e4m3 code, the
 * product y = x * fl(1/s) may stand in for the IEEE quotient fl(x / s) unless
 * y lies within 4 binary32 ulps of an e4m3 rounding midpoint (low 20
 * mantissa bits 0x80000 in the normal range), below 2^-6, or 1/s is not
 * finite.  For every bf16 x and N scales (half of them amax / 448 for a
 * bf16 amax, half arbitrary normal binary32), the code of the stand-in must
 * equal the code of the quotient.  With WINDOW = 0 (the midpoint alone) some
 * must differ: that shows the check can fail.
 * Usage: e4m3_shortcut N WINDOW; prints "pairs mismatches" and exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f32(uint32_t b) { float v; memcpy(&v, &b, 4); return v; }
static uint32_t bits(float v) { uint32_t b; memcpy(&b, &v, 4); return b; }

/* e4m3 (OCP, max 448): round to nearest even, saturate, keep the sign of zero */
static uint32_t e4m3(float v) {
  const uint32_t sign = (bits(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);
  const uint32_t b = bits(a);
  return sign | (((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3));
}

static int needs_division(float y, float r, uint32_t window) {
  const uint32_t yb = bits(y) & 0x7FFFFFFFu;
  if (!(r < INFINITY)) return 1;
  return yb < 0x3C800000u || ((yb & 0xFFFFFu) - (0x80000u - window)) < 2u * window + 1u;
}

int main(int argc, char** argv) {
  const int n = argc > 1 ? atoi(argv[1]) : 1000;
  const uint32_t window = argc > 2 ? (uint32_t)atoi(argv[2]) : 4u;
  uint64_t st = 88172645463325252ull;
  long pairs = 0, bad = 0;
  for (int it = 0; it < n; ++it) {
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    volatile float s;
    if (it % 2 == 0) {
      const float amax = f32((uint32_t)(st & 0x7FFF0000u));
      if (!(amax > 0.0f) || !(amax < INFINITY)) continue;
      s = amax / 448.0f;
    } else {
      s = f32((uint32_t)(st % (0x7F000000u - 0x00800000u)) + 0x00800000u);
    }
    if (!(s > 0.0f) || !(s < INFINITY)) continue;
    volatile float r = 1.0f / s;
    for (uint32_t xb = 0; xb < 65536; ++xb) {
      const float x = f32(xb << 16);
      if (!(fabsf(x) < INFINITY)) continue;
      volatile float q = x / s;
      if (!(fabsf(q) < INFINITY)) continue;
      volatile float y = x * r;
      const float stand_in = needs_division(y, r, window) ? q : y;
      ++pairs;
      if (e4m3(stand_in) != e4m3(q)) ++bad;
    }
  }
  printf("%ld %ld\n", pairs, bad);
  return 0;
}
