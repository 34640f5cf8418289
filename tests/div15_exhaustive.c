// Exhaustive check of an identity the quantize kernel relies on: for every
// non-negative finite fp32 d, the corrected product
//   q' = fma(fma(-15, q, d), y, q),  q = d * y,  y = RN(1/15) = 0x1.111112p-4
// equals the IEEE quotient d / 15 bit for bit.  Built and run by
// tests/test_kernel_identities.py (about 2^31 cases, tens of seconds).
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <math.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
int main(void) {
  volatile float fifteen = 15.0f;
  const float y = 1.0f / fifteen;
  if (u(y) != 0x3D888889u) { printf("RN(1/15) = %a, expected 0x1.111112p-4\n", y); return 2; }
  uint64_t bad = 0;
  for (uint32_t b = 0; b < 0x7F800000u; ++b) {
    const float d = f(b);
    const float want = d / fifteen;
    const float q = d * y;
    const float r = fmaf(-15.0f, q, d);
    const float got = fmaf(r, y, q);
    if (u(got) != u(want)) { if (bad < 5) printf("d=%a want=%a got=%a\n", d, want, got); ++bad; }
  }
  printf("mismatches: %llu of %u\n", (unsigned long long)bad, 0x7F800000u);
  return bad != 0;
}
