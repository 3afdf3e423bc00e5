/* Host check of the activation quotient used by the fused W4A8 decode
 * quantizer: for s = RN(amax / 127) with 2^-64 <= amax <= 2^100, r = RN(1/s)
 * and any |v| <= amax, RN(y + RN(v - s y) r) with y = RN(v r) (both outer
 * steps single fmas) equals the IEEE quotient RN(v / s).  Cases: the
 * neighbourhood (+-40 ulps, both signs) of every half-integer and integer
 * multiple of s up to 127.5, plus random v, for pseudo-random scales
 * (a quarter of them powers of two).  Exit status 0 when every case agrees. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float quotient_rcp(float v, float s, float r) {
  const float y = v * r;
  const float e = fmaf(-s, y, v);
  return fmaf(e, r, y);
}

static uint64_t state = 88172645463325252ull;
static uint32_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (uint32_t)state;
}
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static long checked, mismatched;
static void check(float v, float s, float r) {
  const float a = v / s, b = quotient_rcp(v, s, r);
  ++checked;
  if (to_bits(a) != to_bits(b) && !(a == 0.0f && b == 0.0f)) {
    if (mismatched < 5) printf("v=%a s=%a quotient=%a rcp-form=%a\n", v, s, a, b);
    ++mismatched;
  }
}

int main(int argc, char **argv) {
  const long scales = argc > 1 ? atol(argv[1]) : 2000;
  for (long t = 0; t < scales; ++t) {
    float amax = ldexpf(1.0f + (next() & 0x7FFFFF) / 8388608.0f, (int)(next() % 165) - 64);
    if (t % 4 == 0) amax = ldexpf(1.0f, (int)(next() % 165) - 64);
    const float s = amax / 127.0f, r = 1.0f / s;
    for (int h2 = 1; h2 <= 255; ++h2) {
      const uint32_t c = to_bits((float)(h2 * 0.5) * s);
      for (int d = -40; d <= 40; ++d) {
        const float v = from_bits(c + (uint32_t)d);
        if (fabsf(v) <= amax) { check(v, s, r); check(-v, s, r); }
      }
    }
    for (int i = 0; i < 200; ++i) {
      const float v = amax * ((float)(next() & 0xFFFFFF) / 16777216.0f);
      check(v, s, r);
      check(-v, s, r);
    }
  }
  printf("checked %ld, mismatched %ld\n", checked, mismatched);
  return mismatched != 0;
}
