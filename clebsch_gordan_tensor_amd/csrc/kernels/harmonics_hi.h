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

}  // namespace e3k
