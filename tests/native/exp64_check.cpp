// Host-side accuracy sweep of isd::exp_nonpos (the samplers' float64 exp)
// against the C library's exp.  Prints: worst relative error over normal
// results, worst absolute error over subnormal results, and the special cases.
#include <cmath>
#include <cstdio>
#include <limits>

#include "exp64.hpp"

int main() {
  double tab[64];
  for (int j = 0; j < 64; ++j) tab[j] = std::exp2(j / 64.0);
  double worst_rel = 0.0, worst_abs_sub = 0.0;
  const long n = 4000000;
  for (long i = 0; i <= n; ++i) {
    const double t = -746.0 * static_cast<double>(i) / static_cast<double>(n);
    const double a = isd::exp_nonpos(t, tab), b = std::exp(t);
    if (b >= std::numeric_limits<double>::min()) {
      const double e = std::fabs(a - b) / b;
      if (e > worst_rel) worst_rel = e;
    } else {
      const double e = std::fabs(a - b);
      if (e > worst_abs_sub) worst_abs_sub = e;
    }
  }
  std::printf("worst_rel %.6e\n", worst_rel);
  std::printf("worst_abs_subnormal %.6e\n", worst_abs_sub);
  std::printf("exp0 %.17g\n", isd::exp_nonpos(0.0, tab));
  std::printf("exp_minus_tiny %.17g\n", isd::exp_nonpos(-1e-300, tab));
  std::printf("exp_minus_inf %.17g\n", isd::exp_nonpos(-INFINITY, tab));
  // the difference of two -inf logits (a row with no finite entry) is NaN: also 0
  std::printf("exp_nan %.17g\n", isd::exp_nonpos(-INFINITY - -INFINITY, tab));
  std::printf("exp_minus_800 %.17g\n", isd::exp_nonpos(-800.0, tab));
  std::printf("exp_minus_745_3 %.17g\n", isd::exp_nonpos(-745.3, tab));
  std::printf("exp_minus_1 %.17g %.17g\n", isd::exp_nonpos(-1.0, tab), std::exp(-1.0));
  return 0;
}
