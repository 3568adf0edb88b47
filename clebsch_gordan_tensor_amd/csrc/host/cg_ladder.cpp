// Ladder-operator construction of Clebsch-Gordan blocks (see cg_ladder.h).
#include "cg_ladder.h"

#include <cmath>
#include <complex>
#include <cstdlib>

namespace e3 {
namespace {

// Matrix elements of the ladder operators on |l m>:
//   J_+ |l m> = c_plus(l, m) |l m+1>,  J_- |l m> = c_minus(l, m) |l m-1>.
double c_plus(int l, int m) { return std::sqrt(double(l * (l + 1) - m * (m + 1))); }
double c_minus(int l, int m) { return std::sqrt(double(l * (l + 1) - m * (m - 1))); }

using cplx = std::complex<double>;

// Row r = real index m (shifted by +l), column = complex index m'.
// Real harmonics:  m > 0: (Y^{-m} + (-1)^m Y^m)/sqrt2;  m = 0: Y^0;
//                  m < 0: i (Y^m - (-1)^m Y^{-m})/sqrt2.
std::vector<cplx> real_basis(int l) {
  const int n = 2 * l + 1;
  const double s = 1.0 / std::sqrt(2.0);
  std::vector<cplx> U(size_t(n) * n, cplx(0, 0));
  for (int m = -l; m <= l; ++m) {
    const int r = m + l;
    const double sg = (std::abs(m) % 2) ? -1.0 : 1.0;
    if (m == 0) {
      U[r * n + l] = 1.0;
    } else if (m > 0) {
      U[r * n + (l - m)] = s;
      U[r * n + (l + m)] = sg * s;
    } else {
      U[r * n + (l + m)] = cplx(0, s);
      U[r * n + (l - m)] = cplx(0, -sg * s);
    }
  }
  return U;
}

}  // namespace

bool cg_complex_block(int l1, int l2, int L, std::vector<double>& out) {
  if (l1 < 0 || l2 < 0 || L < std::abs(l1 - l2) || L > l1 + l2) return false;
  const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, nL = 2 * L + 1;
  out.assign(size_t(nL) * n1 * n2, 0.0);
  auto at = [&](int M, int m1, int m2) -> double& {
    return out[(size_t(M + L) * n1 + (m1 + l1)) * n2 + (m2 + l2)];
  };

  // Top state |L L> = sum_m V_m |m, L-m>, m in [lo, hi].  The J^2 equation
  // of Appendix G.2 gives, for each m,
  //   L(L+1) V_m = d(m) V_m + a(m) V_{m-1} + b(m) V_{m+1},
  //   d(m) = l1(l1+1) + l2(l2+1) + 2 m (L-m),
  //   a(m) = c_plus(l1, m-1) c_minus(l2, L-m+1),
  //   b(m) = c_minus(l1, m+1) c_plus(l2, L-m-1),
  // solved upward from V_lo = 1 (b(m) != 0 for lo <= m < hi).
  const int lo = std::max(-l1, L - l2), hi = std::min(l1, L + l2);
  std::vector<double> V(size_t(hi - lo + 1), 0.0);
  V[0] = 1.0;
  for (int m = lo; m < hi; ++m) {
    const double d = l1 * (l1 + 1) + l2 * (l2 + 1) + 2.0 * m * (L - m);
    const double prev = (m > lo) ? V[m - 1 - lo] * c_plus(l1, m - 1) * c_minus(l2, L - m + 1) : 0.0;
    const double b = c_minus(l1, m + 1) * c_plus(l2, L - m - 1);
    V[m + 1 - lo] = ((L * (L + 1) - d) * V[m - lo] - prev) / b;
  }
  double nrm = 0.0;
  for (double v : V) nrm += v * v;
  nrm = std::sqrt(nrm);
  const double sgn = (V[l1 - lo] < 0) ? -1.0 : 1.0;  // m1 = l1 is always in range
  for (int m = lo; m <= hi; ++m) at(L, m, L - m) = sgn * V[m - lo] / nrm;

  // Lower: |L M-1> = J_- |L M> / c_minus(L, M).
  for (int M = L; M > -L; --M) {
    const double inv = 1.0 / c_minus(L, M);
    for (int m1 = -l1; m1 <= l1; ++m1) {
      const int m2 = M - m1;
      if (m2 < -l2 || m2 > l2) continue;
      const double v = at(M, m1, m2);
      if (v == 0.0) continue;
      if (m1 > -l1) at(M - 1, m1 - 1, m2) += v * c_minus(l1, m1) * inv;
      if (m2 > -l2) at(M - 1, m1, m2 - 1) += v * c_minus(l2, m2) * inv;
    }
  }
  return true;
}

bool cg_real_block(int l1, int l2, int L, std::vector<double>& out) {
  std::vector<double> Cc;
  if (!cg_complex_block(l1, l2, L, Cc)) return false;
  const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, nL = 2 * L + 1;
  const std::vector<cplx> U1 = real_basis(l1), U2 = real_basis(l2), UL = real_basis(L);
  const bool odd = (l1 + l2 + L) % 2 != 0;
  out.assign(size_t(nL) * n1 * n2, 0.0);
  // T[M][a][b] = sum U_L[M][M'] C[M'][a'][b'] conj(U1[a][a']) conj(U2[b][b'])
  for (int M = 0; M < nL; ++M)
    for (int a = 0; a < n1; ++a)
      for (int b = 0; b < n2; ++b) {
        cplx t(0, 0);
        for (int Mp = 0; Mp < nL; ++Mp) {
          if (UL[M * nL + Mp] == cplx(0, 0)) continue;
          for (int ap = 0; ap < n1; ++ap) {
            if (U1[a * n1 + ap] == cplx(0, 0)) continue;
            for (int bp = 0; bp < n2; ++bp) {
              const double c = Cc[(size_t(Mp) * n1 + ap) * n2 + bp];
              if (c == 0.0 || U2[b * n2 + bp] == cplx(0, 0)) continue;
              t += UL[M * nL + Mp] * c * std::conj(U1[a * n1 + ap]) * std::conj(U2[b * n2 + bp]);
            }
          }
        }
        double v = odd ? t.imag() : t.real();
        if (std::abs(v) < 1e-13) v = 0.0;
        out[(size_t(M) * n1 + a) * n2 + b] = v;
      }
  return true;
}

}  // namespace e3
