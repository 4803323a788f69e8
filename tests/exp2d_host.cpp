// Host build of the acceptance's float64 2^y (isd_exp2d.hpp) against long
// double exp2l: prints the worst relative error over a seeded sweep and the
// special values, one "name value" pair per line.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "isd_exp2d.hpp"

static uint64_t splitmix(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int main() {
  uint64_t s = 12345;
  double worst = 0.0, worst_y = 0.0;
  for (int i = 0; i < 2000000; ++i) {
    const double r = (double)(splitmix(s) >> 11) * 0x1.0p-53;
    // half the arguments in the sampler's range [-60, 0], half in [-1022, 1023]
    const double y = (i & 1) ? -60.0 * r : -1022.0 + 2045.0 * r;
    const long double ref = exp2l((long double)y);
    const double got = idlm::exp2d(y);
    const double rel = (double)fabsl(((long double)got - ref) / ref);
    if (rel > worst) { worst = rel; worst_y = y; }
  }
  printf("worst_rel %.6e\nworst_y %.17g\n", worst, worst_y);
  // exp2t over the same sweep, from its 64-entry table
  double tab[64];
  for (int j = 0; j < 64; ++j) tab[j] = idlm::exp2t_entry(j, idlm::kExp2Coef);
  s = 12345;
  double worst_t = 0.0;
  for (int i = 0; i < 2000000; ++i) {
    const double r = (double)(splitmix(s) >> 11) * 0x1.0p-53;
    const double y = (i & 1) ? -60.0 * r : -1022.0 + 2045.0 * r;
    const long double ref = exp2l((long double)y);
    const double got = idlm::exp2t(y, tab, idlm::kExp2Coef);
    const double rel = (double)fabsl(((long double)got - ref) / ref);
    if (rel > worst_t) worst_t = rel;
  }
  printf("worst_rel_t %.6e\n", worst_t);
  printf("t_at_0 %.17g\n", idlm::exp2t(0.0, tab, idlm::kExp2Coef));
  printf("t_at_m1 %.17g\n", idlm::exp2t(-1.0, tab, idlm::kExp2Coef));
  printf("t_at_m1075 %.17g\n", idlm::exp2t(-1075.5, tab, idlm::kExp2Coef));
  printf("t_at_nan %.17g\n", idlm::exp2t(NAN, tab, idlm::kExp2Coef));
  // exp2t64 (argument 64 y, scaled coefficients): bit-identical to exp2t for
  // y <= 0.  Sweep: the sampler's form y = d * c with d a difference of two
  // bf16-like values and c a random log2(e)/T, plus the whole range down to
  // past the underflow, and the special values.
  s = 777;
  long mism = 0, count = 0;
  auto same = [&](double y) {
    const double a = idlm::exp2t(y, tab, idlm::kExp2Coef);
    const double b = idlm::exp2t64(y * 64.0, tab, idlm::kExp2Coef64);
    uint64_t ua, ub;
    memcpy(&ua, &a, 8);
    memcpy(&ub, &b, 8);
    mism += ua != ub;
    ++count;
  };
  for (int i = 0; i < 2000000; ++i) {
    const double r = (double)(splitmix(s) >> 11) * 0x1.0p-53;
    const double r2 = (double)(splitmix(s) >> 11) * 0x1.0p-53;
    const double r3 = (double)(splitmix(s) >> 11) * 0x1.0p-53;
    auto bf16 = [](double x) {
      const float f = (float)x;
      uint32_t bits;
      memcpy(&bits, &f, 4);
      bits &= 0xFFFF0000u;
      float g;
      memcpy(&g, &bits, 4);
      return (double)g;
    };
    const double m = bf16(20.0 * r3 - 10.0);         // the row maximum
    const double l = bf16(m - 30.0 * r);              // an element at or below it
    const double c = 1.4426950408889634 / (0.05 + 4.0 * r2);
    if (l <= m) same((l - m) * c);
    same(-1120.0 * r);
  }
  const double specials[] = {0.0, -0.0, -1e-300, -0x1.0p-1074, -1.0 / 128, -1.0 / 64, -0.5,
                             -1022.0, -1074.0, -1075.5, -1100.0, -1e6, -INFINITY, NAN};
  for (double y : specials) same(y);
  printf("t64_mismatch %ld\nt64_count %ld\n", mism, count);
  printf("at_0 %.17g\n", idlm::exp2d(0.0));
  printf("at_1 %.17g\n", idlm::exp2d(1.0));
  printf("at_m1 %.17g\n", idlm::exp2d(-1.0));
  printf("at_half %.17g\n", idlm::exp2d(0.5));
  printf("at_m1074 %.17g\n", idlm::exp2d(-1074.0));
  printf("at_m1075 %.17g\n", idlm::exp2d(-1075.5));
  printf("at_minf %.17g\n", idlm::exp2d(-INFINITY));
  printf("at_nan %.17g\n", idlm::exp2d(NAN));
  printf("at_1024 %.17g\n", idlm::exp2d(1024.0));
  return 0;
}
