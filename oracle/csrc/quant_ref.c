/*
 * Plain C statement of the per-row FP8 E4M3 quantisation, for sweeps too large
 * for numpy (test infrastructure: part of the CPU oracle; only tests/, smoke()
 * and the bench's cpu_baseline may load it). It is the same definition as
 * oracle/quant.py, written again step by step and checked against it:
 *
 *   s = fl32(max |x| / 448); quotient = fl32(x / s) (x itself when s == 0);
 *   code = nearest e4m3fn value of the quotient clamped to +-448, ties to the
 *   even mantissa, sign kept.
 *
 * Method: per-token quantisation of the HunyuanVideo1.5 BF16->FP8 retrospective
 * (aigcage.com, section 3.1) with the scale rule of the Stable Diffusion 3.5 FP8
 * page (dn008.com.cn, FP8 section, steps 1-3) using 448 as the format maximum.
 * Build with plain IEEE float arithmetic: no -ffast-math, -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* nearest e4m3fn code of a finite float, ties to even, saturating at 448 */
static uint8_t encode_e4m3fn(float v) {
  double a = fabs((double)v);
  int negative = signbit(v) ? 1 : 0;
  int code;
  if (a > 448.0) a = 448.0;
  if (a < ldexp(1.0, -6)) {
    code = (int)nearbyint(a * 512.0); /* subnormal grid M * 2^-9; M == 8 is code 0x08 */
  } else {
    int e;
    double mant;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;       /* a = g * 2^e, g in [1, 2) */
    mant = nearbyint((ldexp(a, -e) - 1.0) * 8.0);
    if (mant == 8.0) {
      e += 1;
      mant = 0.0;
    }
    code = ((e + 7) << 3) | (int)mant;
  }
  return (uint8_t)(code | (negative << 7));
}

uint8_t oracle_encode_e4m3fn(float v) { return encode_e4m3fn(v); }

void oracle_quant_rows_bf16(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* scale) {
  int64_t r;
#pragma omp parallel for schedule(dynamic, 8)
  for (r = 0; r < rows; ++r) {
    const uint16_t* xr = x + r * cols;
    uint8_t* qr = q + r * cols;
    volatile float f448 = 448.0f;
    float amax = 0.0f, s;
    int64_t k;
    for (k = 0; k < cols; ++k) {
      float v = fabsf(bf16_to_f32(xr[k]));
      if (v > amax) amax = v;
    }
    s = amax / f448;
    scale[r] = s;
    for (k = 0; k < cols; ++k) {
      float v = bf16_to_f32(xr[k]);
      float quotient = (s == 0.0f) ? v : v / s;
      qr[k] = encode_e4m3fn(quotient);
    }
  }
}
