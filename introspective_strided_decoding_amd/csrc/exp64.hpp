// exp(t) for t <= 0 in float64 by Tang's table-driven method (P. T. P. Tang,
// "Table-driven implementation of the exponential function in IEEE
// floating-point arithmetic", ACM TOMS 15(2), 1989), specialised to the
// arguments the samplers need: t = logit - (a max over the same logits), so
// t <= 0 and no overflow handling is needed.
//
//   n = rint(t * 64 / ln 2),  n = 64 m + j  (0 <= j < 64); n is formed by
//                              adding 1.5 * 2^52 in the same fma that scales t
//                              (the sum's low word then holds n), which saves
//                              the rounding and conversion instructions
//   r = t - n * (ln 2 / 64)   (|r| <= ln 2 / 128; ln 2 / 64 split as hi + lo
//                              with hi's low 17 mantissa bits zero, so n * hi
//                              is exact for |n| < 2^17)
//   exp(t) = 2^m * 2^(j/64) * p(r),  p = degree-5 Taylor polynomial of e^r
//                              (truncation below 3.5e-17 for |r| <= ln 2 / 128)
//
// The 64 values 2^(j/64) live in a caller-provided table (LDS in the
// kernels).  Arguments are clamped to -746 first, where 2^m falls below half
// the smallest subnormal, so -inf and deeper arguments give 0 without a
// branch (NaN arguments are not supported).  Relative error stays within a
// few units in the last place.
#pragma once

#include <hip/hip_runtime.h>

namespace isd {

constexpr double kExpInvStep = 0x1.71547652b82fep+6;     // 64 / ln 2
constexpr double kExpStepHi = 0x1.62e42fefa0000p-7;      // ln 2 / 64, high part
constexpr double kExpStepLo = 0x1.cf79abc9e3b3ap-46;     // ln 2 / 64 - high part
constexpr double kExpClamp = -746.0;

constexpr double kExpShifter = 0x1.8p52;                // 1.5 * 2^52

__host__ __device__ inline double exp_nonpos(double t, const double* __restrict__ tab64) {
  t = fmax(t, kExpClamp);
  // |t * 64 / ln 2| < 2^17, so the shifted sum lies in [2^52, 2^53), where the
  // spacing is 1: it is rounded to the nearest integer, held two's-complement
  // in the low word of the mantissa
  const double k = fma(t, kExpInvStep, kExpShifter);
  const double n = k - kExpShifter;
  unsigned long long kb;
  __builtin_memcpy(&kb, &k, sizeof(kb));
  const int ni = static_cast<int>(static_cast<unsigned int>(kb));
  const int j = ni & 63;
  const int m = ni >> 6;                                 // floor(n / 64)
  const double r = fma(-n, kExpStepLo, fma(-n, kExpStepHi, t));
  double p = 1.0 / 120.0;
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(tab64[j] * p, m);
}

}  // namespace isd
