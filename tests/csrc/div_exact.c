/* Host check of the division identities the bulk quantization kernel uses
 * in place of IEEE division (write.hip, div_bf16 / scale_zero_recip), on the
 * host's IEEE binary32 arithmetic with fused multiply-add:
 *   (1) for y = RN(1/s), q0 = RN(c*y), r = fma(-s, q0, c): fma(r, y, q0) is
 *       RN(c/s), for every binary32 significand of c and every bfloat16
 *       significand of s, with c/s spanning [1/4, 4);
 *   (2) for y0 within 2 ulp of 1/s: fma(fma(-s, y0, 1), y0, y0) is RN(1/s),
 *       for every bfloat16 significand of s.
 * Exponents only scale these results while no operand or residual leaves
 * the normal range, which the kernel checks before taking this path.
 * Prints the mismatch counts; exits non-zero on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t bits(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }

int main(void) {
  long bad_div = 0, bad_rcp = 0;
#pragma omp parallel for reduction(+ : bad_div) schedule(dynamic)
  for (int job = 0; job < 512; ++job) {
    const uint32_t sm = job & 127, se = (job >> 7) & 1, ce = job >> 8;
    volatile float s = f32(((127u + se) << 23) | (sm << 16));
    volatile float one = 1.0f;
    const float y = one / s;
    for (uint32_t cm = 0; cm < (1u << 23); ++cm) {
      const float c = f32(((127u + ce) << 23) | cm);
      volatile float vc = c;
      const float ex = vc / s;
      const float q0 = c * y;
      const float r = fmaf(-s, q0, c);
      const float q = fmaf(r, y, q0);
      bad_div += bits(q) != bits(ex);
    }
  }
  for (uint32_t sm = 0; sm < 128; ++sm) {
    volatile float s = f32((127u << 23) | (sm << 16));
    volatile float one = 1.0f;
    const float ex = one / s;
    for (int d = -2; d <= 2; ++d) {
      const float y0 = f32(bits(ex) + d);
      const float y1 = fmaf(fmaf(-s, y0, 1.0f), y0, y0);
      bad_rcp += bits(y1) != bits(ex);
    }
  }
  printf("division mismatches %ld of %ld, reciprocal mismatches %ld of %d\n", bad_div, 512L << 23, bad_rcp,
         128 * 5);
  return (bad_div || bad_rcp) ? 1 : 0;
}
