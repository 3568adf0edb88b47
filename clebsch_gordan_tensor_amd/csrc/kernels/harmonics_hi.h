// Real harmonics of degree 0..LMAX (LMAX <= 6) of a unit vector, degrees
// 0..3 from their closed forms and 4..6 by the library's own recursion: the
// coupled product of Y_1 and Y_{L-1} through the real (1, L-1 -> L) block is
// kappa_L Y_L (the Gaunt relation for an even path; e3j G.1-G.2 build the
// harmonics and the coefficients from the same ladder structure), with the
// records and 1/kappa_L generated and checked at build time (gen_cg_table).
// The recursion is unrolled at compile time.
#pragma once

#include "common.h"

namespace e3k {

template <int LMAX>
__device__ __forceinline__ void harmonics_bank(float x, float y, float z,
                                               float (&Y)[(LMAX + 1) * (LMAX + 1)]) {
  static_assert(LMAX <= kShLmax, "degree above the generated recursion");
  sfor<0, (LMAX < 3 ? LMAX : 3) + 1>([&](auto l) { harmonics_l<l>(x, y, z, Y + l * l); });
  sfor<4, LMAX + 1>([&](auto L) {
    constexpr int o = L * L, o1 = (L - 1) * (L - 1);
#pragma unroll
    for (int M = 0; M < 2 * L + 1; ++M) Y[o + M] = 0.0f;
    sfor<0, kShRecCnt[L]>([&](auto r) {
      constexpr CgRec R = kShRec[kShRecOff[L] + r];
      Y[o + R.M] = fmaf(R.c * Y[1 + R.m1], Y[o1 + R.m2], Y[o + R.M]);
    });
#pragma unroll
    for (int M = 0; M < 2 * L + 1; ++M) Y[o + M] *= kShInvKappa[L];
  });
}

// Gradient with respect to the unit vector u = (x, y, z) of
// sum_{l <= LMAX, m} w(l*l + m) Y_lm(u), by forward-mode derivatives of the
// same polynomials as harmonics_bank (degrees 0..3 closed form, 4..LMAX by
// the coupling recursion).  Only the previous degree is kept while the
// recursion climbs, and each degree is contracted with w as it is made.
template <int LMAX, class WF>
__device__ __forceinline__ void harmonics_grad_bank(float x, float y, float z, WF w, float& g0,
                                                    float& g1, float& g2) {
  static_assert(LMAX <= kShLmax, "degree above the generated recursion");
  constexpr int L3 = LMAX < 3 ? LMAX : 3;
  const Dual3 X(x, 1.0f, 0.0f, 0.0f), Yd(y, 0.0f, 1.0f, 0.0f), Z(z, 0.0f, 0.0f, 1.0f);
  Dual3 y1[3];
  harmonics_l<1>(X, Yd, Z, y1);
  Dual3 prev[2 * LMAX + 1];
  auto add = [&](int k, const Dual3& h) {
    const float c = w(k);
    g0 = fmaf(c, h.d0, g0);
    g1 = fmaf(c, h.d1, g1);
    g2 = fmaf(c, h.d2, g2);
  };
  sfor<0, L3 + 1>([&](auto l) {
    Dual3 h[2 * l + 1];
    harmonics_l<l>(X, Yd, Z, h);
#pragma unroll
    for (int m = 0; m < 2 * l + 1; ++m) {
      add(l * l + m, h[m]);
      if constexpr (l == L3) prev[m] = h[m];
    }
  });
  sfor<4, LMAX + 1>([&](auto L) {
    Dual3 cur[2 * L + 1];
    sfor<0, kShRecCnt[L]>([&](auto r) {
      constexpr CgRec R = kShRec[kShRecOff[L] + r];
      cur[R.M] = cur[R.M] + (R.c * y1[R.m1]) * prev[R.m2];
    });
#pragma unroll
    for (int M = 0; M < 2 * L + 1; ++M) {
      cur[M] = kShInvKappa[L] * cur[M];
      add(L * L + M, cur[M]);
      prev[M] = cur[M];
    }
  });
}

}  // namespace e3k
