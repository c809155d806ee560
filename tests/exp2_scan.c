/* Exhaustive error scan of the VALU cubic exp2 (exp2_poly.h), every fp32 x in [-126, 8].
 *
 * The evaluation repeats the kernel's fp32 steps (attn_fwd_bf16.hip, exp2_poly): clamp at
 * -126, n = floor(x), f = x - n, p = fma(f, fma(f, fma(f, C3, C2), C1), 1) with fused
 * multiply-adds (v_fma_f32 rounds once, as C's fmaf does), then n added to the exponent
 * bits.  Each result is compared with 2^x in double precision.
 * Prints: the number of values scanned and the largest relative error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "exp2_poly.h"

static float poly_exp2(float x) {
  x = fmaxf(x, -126.0f);
  const float n = floorf(x);
  const float f = x - n;
  const float p = fmaf(f, fmaf(f, fmaf(f, ATTN_EXP2_C3, ATTN_EXP2_C2), ATTN_EXP2_C1), 1.0f);
  int32_t b;
  memcpy(&b, &p, 4);
  b += (int32_t)n << 23;
  float r;
  memcpy(&r, &b, 4);
  return r;
}

int main(void) {
  /* bit patterns of [+0, 8] and of [-0, -126] */
  const int64_t n_pos = 0x41000000LL + 1, n_neg = 0x42FC0000LL + 1;
  const int64_t total = n_pos + n_neg;
  double worst = 0.0;
#pragma omp parallel for reduction(max : worst) schedule(static, 1 << 20)
  for (int64_t i = 0; i < total; ++i) {
    const uint32_t bits = i < n_pos ? (uint32_t)i : 0x80000000u + (uint32_t)(i - n_pos);
    float x;
    memcpy(&x, &bits, 4);
    const double exact = exp2((double)x);
    const double rel = fabs((double)poly_exp2(x) / exact - 1.0);
    if (rel > worst) worst = rel;
  }
  printf("%lld %.9e\n", (long long)total, worst);
  return 0;
}
