// exp2d: 2^y in float64 for the acceptance's sampling weights.
//
// Written from the mathematics, for host and device alike (the host build is
// what the CPU tests check against long double):
//   y = n + f with n = nearest integer to y, |f| <= 1/2 (f exact);
//   2^f = e^(f ln 2) = sum_k (ln 2)^k f^k / k!, the Taylor series cut after
//   k = 13: the remainder is below (ln2 / 2)^14 / 14! ~ 4.3e-18 relative;
//   2^y = 2^f * 2^n by an exponent shift (ldexp).
// Horner's rule in f with coefficients (ln 2)^k / k! folded at compile time.
// Accuracy: under one unit in the last place for y in [-1022, 1023]; below
// that the result goes subnormal and then to 0 (y <= -1075, and -inf); y is
// clamped into [-1100, 1024] first, so no path branches (a NaN y gives 0).
//
// Device code passes the coefficients in as an argument (Exp2Coef, part of
// the kernel arguments): they then sit in scalar registers and feed the
// FMAs directly instead of being rebuilt from literals at every use.
#pragma once

#include <math.h>

#if defined(__HIPCC__)
#define IDLM_HD __host__ __device__
#else
#define IDLM_HD
#endif

namespace idlm {

namespace exp2d_detail {
constexpr double kLn2 = 0.693147180559945309417232121458176568;
constexpr double fact(int k) { return k <= 1 ? 1.0 : k * fact(k - 1); }
constexpr double ipow(double x, int k) { return k == 0 ? 1.0 : x * ipow(x, k - 1); }
constexpr double coef(int k) { return ipow(kLn2, k) / fact(k); }
}  // namespace exp2d_detail

// (ln 2)^k / k!, k = 0..13.
struct Exp2Coef {
  double c[14];
};

constexpr Exp2Coef kExp2Coef = {{1.0, exp2d_detail::coef(1), exp2d_detail::coef(2),
                                 exp2d_detail::coef(3), exp2d_detail::coef(4),
                                 exp2d_detail::coef(5), exp2d_detail::coef(6),
                                 exp2d_detail::coef(7), exp2d_detail::coef(8),
                                 exp2d_detail::coef(9), exp2d_detail::coef(10),
                                 exp2d_detail::coef(11), exp2d_detail::coef(12),
                                 exp2d_detail::coef(13)}};

IDLM_HD inline double exp2d(double y, const Exp2Coef& k) {
  y = fmin(fmax(y, -1100.0), 1024.0);
  const double n = rint(y);
  const double f = y - n;  // exact
  double p = k.c[13];
  p = fma(p, f, k.c[12]);
  p = fma(p, f, k.c[11]);
  p = fma(p, f, k.c[10]);
  p = fma(p, f, k.c[9]);
  p = fma(p, f, k.c[8]);
  p = fma(p, f, k.c[7]);
  p = fma(p, f, k.c[6]);
  p = fma(p, f, k.c[5]);
  p = fma(p, f, k.c[4]);
  p = fma(p, f, k.c[3]);
  p = fma(p, f, k.c[2]);
  p = fma(p, f, k.c[1]);
  p = fma(p, f, 1.0);
  return ldexp(p, (int)n);
}

IDLM_HD inline double exp2d(double y) { return exp2d(y, kExp2Coef); }

// exp2t: the same 2^y from a table, for the sampler's many exponentials:
//   y = k/64 + r with k the nearest integer to 64 y, |r| <= 1/128 (r exact);
//   2^y = 2^(k >> 6) * 2^((k & 63)/64) * 2^r, the middle factor from `tab`
//   (tab[j] = exp2d(j/64), built by exp2t_entry), 2^r by the Taylor series
//   cut after r^5 (remainder below (ln2/128)^6/6! ~ 3.5e-17 relative).
// About five fewer arithmetic instructions than exp2d; worst relative error
// about three units in the last place.  y is clamped into [-1100, 1024]
// first (a NaN y gives 0).
IDLM_HD inline double exp2t_entry(int j, const Exp2Coef& k) { return exp2d(j / 64.0, k); }

IDLM_HD inline double exp2t(double y, const double* tab, const Exp2Coef& k) {
  y = fmin(fmax(y, -1100.0), 1024.0);
  const double kk = rint(y * 64.0);
  const double r = fma(kk, -0.015625, y);  // exact
  const int ki = (int)kk;
  double p = k.c[5];
  p = fma(p, r, k.c[4]);
  p = fma(p, r, k.c[3]);
  p = fma(p, r, k.c[2]);
  p = fma(p, r, k.c[1]);
  p = fma(p, r, 1.0);
  return ldexp(p * tab[ki & 63], ki >> 6);
}

// exp2t64: exp2t with the argument given as z = 64 y, for callers that fold
// the factor 64 into their own scale and whose y is never positive (a weight
// relative to its row maximum).  With s = z - k = 64 r the polynomial runs
// in s on the coefficients (ln 2)^j / j! / 64^j; every step of it is the
// corresponding step of exp2t scaled by a power of two, so the result is
// bit-identical to exp2t(z / 64) for z <= 0, in two fewer instructions (the
// scaling and the upper clamp).  z is clamped below at -70400 (y = -1100;
// a NaN z gives 0).
struct Exp2Coef64 {
  double c[6];
};

constexpr Exp2Coef64 kExp2Coef64 = {{1.0, exp2d_detail::coef(1) / 64.0,
                                     exp2d_detail::coef(2) / 4096.0,
                                     exp2d_detail::coef(3) / 262144.0,
                                     exp2d_detail::coef(4) / 16777216.0,
                                     exp2d_detail::coef(5) / 1073741824.0}};

IDLM_HD inline double exp2t64(double z, const double* tab, const Exp2Coef64& k) {
  z = fmax(z, -70400.0);
  const double kk = rint(z);
  const double s = z - kk;  // exact, |s| <= 1/2
  const int ki = (int)kk;
  double p = k.c[5];
  p = fma(p, s, k.c[4]);
  p = fma(p, s, k.c[3]);
  p = fma(p, s, k.c[2]);
  p = fma(p, s, k.c[1]);
  p = fma(p, s, 1.0);
  return ldexp(p * tab[ki & 63], ki >> 6);
}

}  // namespace idlm
