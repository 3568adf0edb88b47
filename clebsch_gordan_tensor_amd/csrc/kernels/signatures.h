// Irreps signatures (x, y, output) with specialised, fully unrolled kernels.
// Every x and output irrep carries the same multiplicity C (channel-wise
// product); y is the harmonic bank (multiplicity 1).  Parities: e = +1, o = -1.
//
// kBwdWaves[c] (optional): wavefronts per SIMD the convolution backward is
// compiled for with 2^c channels per lane -- set where the compiler fits that
// occupancy without spilling but its default schedule (after the per-chunk
// staging of the harmonics) would settle lower; 1 leaves the choice to it.
// kStageY (optional, default true): false makes the backward form the
// harmonics per edge in its loop instead of staging them per chunk in LDS
// (the register allocation of the larger signatures fares better so).
#pragma once

#include "common.h"

namespace e3k {

// 0e+1o (x) Y_0..1 -> 0e+1o
struct SigL1 {
  static constexpr int NX = 2, NY = 2, NO = 2;
  static constexpr int kBwdWaves[3] = {3, 3, 3};
  static constexpr Ir X[NX] = {{0, 1}, {1, -1}};
  static constexpr Ir Y[NY] = {{0, 1}, {1, -1}};
  static constexpr Ir O[NO] = {{0, 1}, {1, -1}};
};

// 0e+1o (x) Y_0..3 -> 0e+1o+2e+3o   (MACE-like interaction, 10 paths)
struct SigL1to3 {
  static constexpr int NX = 2, NY = 4, NO = 4;
  static constexpr int kBwdWaves[3] = {3, 3, 1};
  static constexpr Ir X[NX] = {{0, 1}, {1, -1}};
  static constexpr Ir Y[NY] = {{0, 1}, {1, -1}, {2, 1}, {3, -1}};
  static constexpr Ir O[NO] = {{0, 1}, {1, -1}, {2, 1}, {3, -1}};
};

// 0e+1o+2e (x) Y_0..3 -> 0e+1o+2e+3o   (17 paths)
struct SigL2to3 {
  static constexpr int NX = 3, NY = 4, NO = 4;
  static constexpr int kBwdWaves[3] = {3, 1, 1};
  static constexpr Ir X[NX] = {{0, 1}, {1, -1}, {2, 1}};
  static constexpr Ir Y[NY] = {{0, 1}, {1, -1}, {2, 1}, {3, -1}};
  static constexpr Ir O[NO] = {{0, 1}, {1, -1}, {2, 1}, {3, -1}};
};

// 0e+1o+2e+3o (x) Y_0..3 -> 0e+1o+2e+3o   (23 paths)
struct SigL3to3 {
  static constexpr int NX = 4, NY = 4, NO = 4;
  static constexpr Ir X[NX] = {{0, 1}, {1, -1}, {2, 1}, {3, -1}};
  static constexpr Ir Y[NY] = {{0, 1}, {1, -1}, {2, 1}, {3, -1}};
  static constexpr Ir O[NO] = {{0, 1}, {1, -1}, {2, 1}, {3, -1}};
};

// 0e+1o (x) Y_0..3 -> every parity-allowed output up to l = 3, pseudotensors
// included: 0e+1o+1e+2e+2o+3o+3e (13 paths)
struct SigL1to3All {
  static constexpr int NX = 2, NY = 4, NO = 7;
  static constexpr bool kStageY = false;
  static constexpr Ir X[NX] = {{0, 1}, {1, -1}};
  static constexpr Ir Y[NY] = {{0, 1}, {1, -1}, {2, 1}, {3, -1}};
  static constexpr Ir O[NO] = {{0, 1}, {1, -1}, {1, 1}, {2, 1}, {2, -1}, {3, -1}, {3, 1}};
};

// One output block per path (e3j's default) on signature B's paths.
template <class B>
struct PerPath : B {
  static constexpr bool kPerPath = true;
  static constexpr int kBwdWaves[3] = {1, 1, 1};
  static constexpr bool kStageY = false;
};

}  // namespace e3k
