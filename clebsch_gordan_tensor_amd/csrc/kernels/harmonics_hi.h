// Real harmonics of degree 0..LMAX (LMAX <= 8) of a unit vector, degrees
// 0..3 from their closed forms and 4..8 by the library's own recursion: the
// coupled product of Y_1 and Y_{L-1} through the real (1, L-1 -> L) block is
// kappa_L Y_L (the Gaunt relation for an even path; e3j G.1-G.2 build the
// harmonics and the coefficients from the same ladder structure), with the
// records and 1/kappa_L generated and checked at build time (gen_cg_table).
// The recursion is unrolled at compile time.
#pragma once

#include "common.h"

namespace e3k {

// Coefficients of the recursion at degree L in the working precision R.
template <class R, int L, int I>
__device__ __forceinline__ constexpr R sh_rec_c() {
  if constexpr (std::is_same_v<R, double>)
    return kShRecD[kShRecOff[L] + I].c;
  else
    return kShRec[kShRecOff[L] + I].c;
}
template <class R, int L>
__device__ __forceinline__ constexpr R sh_inv_kappa() {
  if constexpr (std::is_same_v<R, double>)
    return kShInvKappaD[L];
  else
    return kShInvKappa[L];
}

template <int LMAX, class R>
__device__ __forceinline__ void harmonics_bank(R x, R y, R z, R (&Y)[(LMAX + 1) * (LMAX + 1)]) {
  static_assert(LMAX <= kShLmax, "degree above the generated recursion");
  sfor<0, (LMAX < 3 ? LMAX : 3) + 1>([&](auto l) { harmonics_l<l>(x, y, z, Y + l * l); });
  sfor<4, LMAX + 1>([&](auto L) {
    constexpr int o = L * L, o1 = (L - 1) * (L - 1);
#pragma unroll
    for (int M = 0; M < 2 * L + 1; ++M) Y[o + M] = R(0);
    sfor<0, kShRecCnt[L]>([&](auto r) {
      constexpr CgRec Q = kShRec[kShRecOff[L] + r];
      Y[o + Q.M] = fma(sh_rec_c<R, L, r>() * Y[1 + Q.m1], Y[o1 + Q.m2], Y[o + Q.M]);
    });
#pragma unroll
    for (int M = 0; M < 2 * L + 1; ++M) Y[o + M] *= sh_inv_kappa<R, L>();
  });
}

// The bank of degree 0..LMAX of the (unnormalised) edge vector (x, y, z) in
// float32 (unit_vector, then the polynomials and the recursion); the zero
// vector gives Y_0 = 1 and 0 above.  The coefficient-table and dense-product
// kernels form it per edge, where fp64 would cost them registers.
template <int LMAX>
__device__ __forceinline__ void harmonics_bank_of_vec(float x, float y, float z,
                                                      float (&Y)[(LMAX + 1) * (LMAX + 1)]) {
  unit_vector(x, y, z);
  harmonics_bank<LMAX>(x, y, z, Y);
}

// The same bank in fp64 on the fp64 direction, rounded once (as the
// specialised convolution kernels' harmonics of degree <= 3).
template <int LMAX>
__device__ __forceinline__ void harmonics_bank_of_vec_f64(float vx, float vy, float vz,
                                                          float (&Y)[(LMAX + 1) * (LMAX + 1)]) {
  double x, y, z;
  unit_dir_f64(vx, vy, vz, x, y, z);
  double h[(LMAX + 1) * (LMAX + 1)];
  harmonics_bank<LMAX>(x, y, z, h);
#pragma unroll
  for (int i = 0; i < (LMAX + 1) * (LMAX + 1); ++i) Y[i] = float(h[i]);
}

// Gradient with respect to the unit vector u = (x, y, z) of
// sum_{l <= LMAX, m} w(l*l + m) Y_lm(u), by forward-mode derivatives of the
// same polynomials as harmonics_bank (degrees 0..3 closed form, 4..LMAX by
// the coupling recursion), in the precision R.  Only the previous degree is
// kept while the recursion climbs, and each degree is contracted with w as
// it is made.
template <int LMAX, class R, class WF>
__device__ __forceinline__ void harmonics_grad_bank(R x, R y, R z, WF w, R& g0, R& g1, R& g2) {
  static_assert(LMAX <= kShLmax, "degree above the generated recursion");
  using D = DualT<R>;
  constexpr int L3 = LMAX < 3 ? LMAX : 3;
  const D X(x, R(1), R(0), R(0)), Yd(y, R(0), R(1), R(0)), Z(z, R(0), R(0), R(1));
  D y1[3];
  harmonics_l<1>(X, Yd, Z, y1);
  D prev[2 * LMAX + 1];
  auto add = [&](int k, const D& h) {
    const R c = R(w(k));
    g0 = fma(c, h.d0, g0);
    g1 = fma(c, h.d1, g1);
    g2 = fma(c, h.d2, g2);
  };
  sfor<0, L3 + 1>([&](auto l) {
    D h[2 * l + 1];
    harmonics_l<l>(X, Yd, Z, h);
#pragma unroll
    for (int m = 0; m < 2 * l + 1; ++m) {
      add(l * l + m, h[m]);
      if constexpr (l == L3) prev[m] = h[m];
    }
  });
  sfor<4, LMAX + 1>([&](auto L) {
    D cur[2 * L + 1];
    sfor<0, kShRecCnt[L]>([&](auto r) {
      constexpr CgRec Q = kShRec[kShRecOff[L] + r];
      cur[Q.M] = cur[Q.M] + (sh_rec_c<R, L, r>() * y1[Q.m1]) * prev[Q.m2];
    });
#pragma unroll
    for (int M = 0; M < 2 * L + 1; ++M) {
      cur[M] = sh_inv_kappa<R, L>() * cur[M];
      add(L * L + M, cur[M]);
      prev[M] = cur[M];
    }
  });
}

}  // namespace e3k
