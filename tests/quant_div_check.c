/* Exhaustive check of the division the activation quantization kernels use
 * for the 1x128 rule (fp32 scale s = max(amax, 1e-4) / 448, code = e4m3 of
 * x / s with x / s an IEEE fp32 division, round to nearest even).
 *
 * The kernels divide once per block, r = 1 / s (IEEE), and per element take
 *   q0 = x * r,  rem = fma(-s, q0, x)  (exact),  q = fma(rem, r, q0),
 * with the sign of x restored for x = -0.  By Markstein's theorem on
 * division by reciprocal and one correction step, q is the correctly rounded
 * quotient wherever no operand or intermediate is subnormal.  This program
 * does not rely on the theorem: for every scale the rule can produce (every
 * bf16 amax, with the 1e-4 floor) and every finite bf16 x with |x| <= the
 * block's floored amax, it compares q with x / s.  Where |x / s| >= 2^-11 the
 * two must be the same fp32 bits; below, both must be under 2^-10 with the
 * same sign, so both encode to the same signed zero (the smallest e4m3
 * subnormal is 2^-9, so everything below 2^-10 rounds to zero).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp quant_div_check.c -lm
 * Exit status 0 and "0 mismatches" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t u_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

int main(void) {
  long long bad = 0, n = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad, n)
  for (int a = 0; a < 0x7F80; ++a) {
    const float amax = f_of((uint32_t)a << 16);
    if (a > 0 && amax < 1e-4f) continue; /* floored: the same scale as amax = 0 */
    volatile float m = amax < 1e-4f ? 1e-4f : amax;
    const float s = m / 448.0f;
    volatile float one = 1.0f;
    const float r = one / s;
    for (uint32_t xb = 0; xb < 0x10000; ++xb) {
      if ((xb & 0x7F80) == 0x7F80) continue; /* inf, nan */
      const float x = f_of(xb << 16);
      if (fabsf(x) > m) continue;
      volatile float q_ref = x / s;
      const float q0 = x * r;
      const float rem = fmaf(-s, q0, x);
      const float q = copysignf(fmaf(rem, r, q0), x);
      int same;
      if (fabsf(q_ref) < 0x1p-11f)
        same = fabsf(q) < 0x1p-10f && signbit(q) == signbit(q_ref);
      else
        same = u_of(q) == u_of(q_ref);
      ++n;
      if (!same) ++bad;
    }
  }
  printf("checked %lld pairs, %lld mismatches\n", n, bad);
  return bad != 0;
}
