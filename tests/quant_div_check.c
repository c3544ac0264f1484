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
 * A second pass covers fp32 inputs (the SwiGLU output h, quantized with the
 * same rule along I): seeded pairs of a random positive fp32 block amax (all
 * exponents) and a random fp32 x with |x| <= the floored amax, the block's
 * largest element itself included, under the same comparison.
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

/* The kernels' quotient and the comparison rule above: 1 when they agree. */
static int agrees(float x, float s, float r) {
  volatile float q_ref = x / s;
  const float q0 = x * r;
  const float rem = fmaf(-s, q0, x);
  const float q = copysignf(fmaf(rem, r, q0), x);
  if (fabsf(q_ref) < 0x1p-11f) return fabsf(q) < 0x1p-10f && signbit(q) == signbit(q_ref);
  return u_of(q) == u_of(q_ref);
}

/* splitmix64: the sample generator of the fp32 pass */
static uint64_t mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static long long fp32_pass(long long *n_out) {
  const long long per = 1 << 14, blocks = 1 << 14; /* 2^28 pairs */
  long long bad = 0, n = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : bad, n)
  for (long long b = 0; b < blocks; ++b) {
    uint64_t st = mix((uint64_t)b * 0x100000001B3ull + 12345);
    /* one block amax per outer step: any positive finite fp32 */
    const uint32_t abits = (uint32_t)(st % 0x7F800000u);
    const float amax = f_of(abits);
    volatile float m = amax < 1e-4f ? 1e-4f : amax;
    const float s = m / 448.0f;
    volatile float one = 1.0f;
    const float r = one / s;
    const uint32_t mbits = u_of(m);
    for (long long i = 0; i < per; ++i) {
      st = mix(st);
      uint32_t xb = i == 0 ? mbits : (uint32_t)(st % ((uint64_t)mbits + 1));
      if (st >> 63) xb |= 0x80000000u;
      ++n;
      if (!agrees(f_of(xb), s, r)) ++bad;
    }
  }
  *n_out = n;
  return bad;
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
      ++n;
      if (!agrees(x, s, r)) ++bad;
    }
  }
  printf("bf16 inputs: checked %lld pairs, %lld mismatches\n", n, bad);
  long long n32 = 0;
  const long long bad32 = fp32_pass(&n32);
  printf("fp32 inputs: checked %lld pairs, %lld mismatches\n", n32, bad32);
  return bad != 0 || bad32 != 0;
}
