/* Exhaustive checks of two fp32 identities the device quantizer relies on.
 *
 * 1. Division by 7: for every non-negative finite fp32 a,
 *        q = a * c;  q' = fma(fma(-q, 7, a), c, q)      (c = fp32(1/7))
 *    equals the correctly rounded a / 7 (division by a constant known in
 *    advance: Brisebarre, Muller and Raina, IEEE Trans. Computers 53(8), 2004).
 * 2. Reciprocal of a group scale: for every positive finite fp16 value s and
 *    any fp32 r0 within two floats of the correctly rounded 1/s (the
 *    hardware reciprocal is documented to within one ulp), one Newton step
 *        e = fma(-s, r0, 1);  r = fma(e, r0, r0)
 *    gives the correctly rounded fp32 1 / s.
 * Exit status 0 and "ok" when both hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* IEEE binary16 bit pattern -> float (exact) */
static float half_to_float(uint16_t h) {
  const int e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else v = ldexpf((float)(m | 0x400), e - 25);
  return (h & 0x8000) ? -v : v;
}

int main(void) {
  const float c = 1.0f / 7.0f;
  unsigned long long bad7 = 0;
#pragma omp parallel for reduction(+ : bad7) schedule(static)
  for (long long i = 0; i <= 0x7F7FFFFFLL; ++i) {
    const float a = f_of((uint32_t)i);
    const volatile float ref = a / 7.0f;
    const float q = a * c;
    const float q1 = fmaf(fmaf(-q, 7.0f, a), c, q);
    if (u_of(q1) != u_of(ref)) bad7++;
  }
  unsigned long long badr = 0, nr = 0;
  for (uint32_t h = 1; h < 0x7C00; ++h) {
    const float s = half_to_float((uint16_t)h);
    const volatile float ref = 1.0f / s;
    const uint32_t u = u_of(ref);
    const uint32_t cand[5] = {u - 2, u - 1, u, u + 1, u + 2};
    for (int k = 0; k < 5; ++k) {
      const float r0 = f_of(cand[k]);
      const float e = fmaf(-s, r0, 1.0f);
      const float r = fmaf(e, r0, r0);
      nr++;
      if (u_of(r) != u) badr++;
    }
  }
  printf("div7 mismatches %llu; reciprocal cases %llu, mismatches %llu\n", bad7, nr, badr);
  if (bad7 == 0 && badr == 0) printf("ok\n");
  return (bad7 == 0 && badr == 0) ? 0 : 1;
}
