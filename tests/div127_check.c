/* Host check of the quantiser's division-free scale: for non-negative finite
 * fp32 m, q1 = RN(m * RN(1/127)), e = fma(-q1, 127, m), q2 = fma(e, RN(1/127), q1)
 * must equal the IEEE quotient RN(m / 127).  argv[1] = stride over the bit
 * patterns (1 = exhaustive).  Prints the mismatch count; exit status 1 if any. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int main(int argc, char** argv) {
  const uint32_t stride = argc > 1 ? (uint32_t)strtoul(argv[1], 0, 10) : 1u;
  const float r = 1.0f / 127.0f;
  uint64_t n = 0, bad = 0;
  for (uint64_t u = 0; u < 0x7f800000u; u += stride) {
    const uint32_t bits = (uint32_t)u;
    float m;
    memcpy(&m, &bits, 4);
    const volatile float ref = m / 127.0f;
    const float q1 = m * r;
    const float e = fmaf(-q1, 127.0f, m);
    const float q2 = fmaf(e, r, q1);
    if (q2 != ref) {
      if (bad < 5) printf("mismatch m=%a ref=%a got=%a\n", m, ref, q2);
      ++bad;
    }
    ++n;
  }
  printf("%llu values, %llu mismatches\n", (unsigned long long)n, (unsigned long long)bad);
  return bad != 0;
}
