/* Exhaustive check of the quantisers' divide-free quotient against the correctly rounded one.
 *
 * For a per-tensor or per-token scale s = fl32(amax / fmax), the GPU quantisers form
 * x / s as q0 = x * r, e = fma(q0, s, -x), q = fma(-e, r, q0) with r = fl32(1 / s), from
 * amax >= 2^-80 on. Over every pair of finite bf16 values (x, amax) with amax >= 2^-80 and
 * |x| <= amax, both signs of x, this program compares q with fl32(x / s) bit for bit and
 * prints, for the fmax given on the command line: the number of pairs, the number where the
 * two differ, the largest magnitude of either among those, and how many of those differ in
 * sign. Build without floating-point contraction (-ffp-contract=off). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t b) {
  const uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  const float fmax = strtof(argv[1], NULL);
  long long pairs = 0, differ = 0, sign_differ = 0;
  float largest = 0.0f;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : pairs, differ, sign_differ) reduction(max : largest)
  for (int a = 1; a < 0x7f80; ++a) {
    const float amax = bf16((uint32_t)a);
    if (amax < 0x1p-80f) continue;
    const float s = amax / fmax;
    const float r = 1.0f / s;
    for (int m = 0; m <= a; ++m) {
      for (int neg = 0; neg < 2; ++neg) {
        const float x = neg ? -bf16((uint32_t)m) : bf16((uint32_t)m);
        const float exact = x / s;
        const float q0 = x * r;
        const float e = fmaf(q0, s, -x);
        const float q = fmaf(-e, r, q0);
        ++pairs;
        if (memcmp(&exact, &q, 4) != 0) {
          ++differ;
          if (signbit(exact) != signbit(q)) ++sign_differ;
          largest = fmaxf(largest, fmaxf(fabsf(exact), fabsf(q)));
        }
      }
    }
  }
  printf("%lld %lld %a %lld\n", pairs, differ, largest, sign_differ);
  return 0;
}
