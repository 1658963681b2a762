/* div6_check.c -- CPU check of the block-scale quotient the quantizers compute on
 * the GPU (device.hpp, div6): for x >= 2^-125, x * RN(1/6) corrected by one fused
 * residual step, RN(q0 + RN(x - 6 q0) * RN(1/6)) with q0 = RN(x * RN(1/6)), equals the
 * correctly rounded quotient x / 6.  fmaf is the single-rounding fused multiply-add
 * (built with -mfma, no contraction elsewhere), as v_fma_f32 is on the GPU.
 * Counts the binary32 bit patterns in [lo, hi] where the two differ. */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float from_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}

static uint32_t to_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

uint64_t div6_mismatches(uint32_t lo, uint32_t hi, uint32_t *first_bad) {
  const float r6 = 1.0f / 6.0f;
  uint64_t bad = 0;
  uint32_t first = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : first)
  for (int64_t i = lo; i <= (int64_t)hi; ++i) {
    const float x = from_bits((uint32_t)i);
    const float q0 = x * r6;
    const float q = fmaf(fmaf(-q0, 6.0f, x), r6, q0);
    if (to_bits(q) != to_bits(x / 6.0f)) {
      bad += 1;
      if ((uint32_t)i < first) first = (uint32_t)i;
    }
  }
  *first_bad = first;
  return bad;
}
