// Build step: writes the compile-time CG record table that the gfx950
// kernels unroll.  For every coupled triple (l1, l2, L) with l1, l2, L <= 3
// it lists the nonzero entries of the real block from cg_real_block(), as
// records (M, m1, m2, c) sorted by (M, m1, m2), with c rounded to fp32; and
// the records that build harmonics of degree 4..6 from lower degrees.
//
// usage: gen_cg_table <output-header>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "cg_ladder.h"

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s <output-header>\n", argv[0]);
    return 2;
  }
  constexpr int LM = 3;
  int off[LM + 1][LM + 1][LM + 1], cnt[LM + 1][LM + 1][LM + 1];
  struct R {
    int M, m1, m2;
    float c;
    double cd;  // the coefficient before rounding to float
  };
  std::vector<R> recs;
  for (int l1 = 0; l1 <= LM; ++l1)
    for (int l2 = 0; l2 <= LM; ++l2)
      for (int L = 0; L <= LM; ++L) {
        off[l1][l2][L] = -1;
        cnt[l1][l2][L] = 0;
        std::vector<double> T;
        if (!e3::cg_real_block(l1, l2, L, T)) continue;
        off[l1][l2][L] = int(recs.size());
        const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
        for (int M = 0; M < 2 * L + 1; ++M)
          for (int a = 0; a < n1; ++a)
            for (int b = 0; b < n2; ++b) {
              const double v = T[(size_t(M) * n1 + a) * n2 + b];
              if (std::abs(v) < 1e-12) continue;
              recs.push_back({M, a, b, float(v), v});
              cnt[l1][l2][L]++;
            }
      }
  FILE* f = std::fopen(argv[1], "w");
  if (!f) {
    std::perror(argv[1]);
    return 1;
  }
  std::fprintf(f,
               "// Generated at build time by gen_cg_table from the ladder-operator CG\n"
               "// construction (cg_ladder.cpp).  Do not edit.\n"
               "#pragma once\n\nnamespace e3k {\n\n"
               "struct CgRec {\n  int M, m1, m2;\n  float c;\n};\n\n"
               "inline constexpr int kTabLmax = %d;\n\n",
               LM);
  auto dump3 = [&](const char* name, int (&a)[LM + 1][LM + 1][LM + 1]) {
    std::fprintf(f, "inline constexpr int %s[%d][%d][%d] = {\n", name, LM + 1, LM + 1, LM + 1);
    for (int i = 0; i <= LM; ++i) {
      std::fprintf(f, "  {");
      for (int j = 0; j <= LM; ++j) {
        std::fprintf(f, "{");
        for (int k = 0; k <= LM; ++k) std::fprintf(f, "%d%s", a[i][j][k], k < LM ? ", " : "");
        std::fprintf(f, "}%s", j < LM ? ", " : "");
      }
      std::fprintf(f, "}%s\n", i < LM ? "," : "");
    }
    std::fprintf(f, "};\n\n");
  };
  dump3("kRecOff", off);
  dump3("kRecCnt", cnt);
  std::fprintf(f, "inline constexpr CgRec kRec[%zu] = {\n", recs.size());
  for (const R& r : recs) std::fprintf(f, "  {%d, %d, %d, %a},\n", r.M, r.m1, r.m2, double(r.c));
  std::fprintf(f, "};\n\n");

  // Harmonics of degree L = 2..kShLmax by the coupling of Y_1 and Y_{L-1}:
  // for the even path (1, L-1 -> L) the coupled product of two harmonics of
  // one vector is kappa_L Y_L (the Gaunt relation), with
  // kappa_L = sqrt(3 (2L-1) / (2L+1)) <1 0 L-1 0 | L 0>.  Records of the real
  // (1, L-1, L) blocks and 1/kappa_L; checked below on random directions.
  constexpr int SL = 8;
  std::vector<R> srec;
  int soff[SL + 1] = {0}, scnt[SL + 1] = {0};
  double inv_kappa[SL + 1] = {0};
  for (int L = 2; L <= SL; ++L) {
    std::vector<double> T, Cc;
    if (!e3::cg_real_block(1, L - 1, L, T) || !e3::cg_complex_block(1, L - 1, L, Cc)) {
      std::fprintf(stderr, "gen_cg_table: (1, %d, %d) does not couple\n", L - 1, L);
      return 1;
    }
    const int n2 = 2 * L - 1;
    const double c00 = Cc[(size_t(L) * 3 + 1) * n2 + (L - 1)];  // <1 0 L-1 0 | L 0>
    inv_kappa[L] = 1.0 / (std::sqrt(3.0 * (2 * L - 1) / (2 * L + 1)) * c00);
    soff[L] = int(srec.size());
    for (int M = 0; M < 2 * L + 1; ++M)
      for (int a = 0; a < 3; ++a)
        for (int b = 0; b < n2; ++b) {
          const double v = T[(size_t(M) * 3 + a) * n2 + b];
          if (std::abs(v) < 1e-12) continue;
          srec.push_back({M, a, b, float(v), v});
          scnt[L]++;
        }
  }
  // self-check in double: sum_m Y_L^2 = 2L+1, Y_L(z) = sqrt(2L+1) e_0, and
  // the recursion reproduces the closed-form cubic at L = 3
  {
    auto bank = [&](double x, double y, double z, std::vector<std::vector<double>>& Y) {
      Y.assign(SL + 1, {});
      Y[0] = {1.0};
      Y[1] = {std::sqrt(3.0) * y, std::sqrt(3.0) * z, std::sqrt(3.0) * x};
      for (int L = 2; L <= SL; ++L) {
        Y[L].assign(2 * L + 1, 0.0);
        for (int r = 0; r < scnt[L]; ++r) {
          const R& q = srec[soff[L] + r];
          Y[L][q.M] += double(q.c) * Y[1][q.m1] * Y[L - 1][q.m2];
        }
        for (double& v : Y[L]) v *= inv_kappa[L];
      }
    };
    std::vector<std::vector<double>> Y;
    unsigned st = 12345u;
    auto rnd = [&]() { st = st * 1664525u + 1013904223u; return (st >> 8) / double(1 << 24) - 0.5; };
    for (int t = 0; t < 200; ++t) {
      double x = rnd(), y = rnd(), z = rnd();
      const double n = std::sqrt(x * x + y * y + z * z);
      x /= n, y /= n, z /= n;
      bank(x, y, z, Y);
      for (int L = 2; L <= SL; ++L) {
        double s2 = 0.0;
        for (double v : Y[L]) s2 += v * v;
        if (std::abs(s2 - (2 * L + 1)) > 1e-5 * (2 * L + 1)) {
          std::fprintf(stderr, "gen_cg_table: harmonic norm check failed at L = %d\n", L);
          return 1;
        }
      }
      const double c3 = std::sqrt(7.0) / 2.0 * z * (2 * z * z - 3 * x * x - 3 * y * y);
      if (std::abs(Y[3][3] - c3) > 1e-5) {
        std::fprintf(stderr, "gen_cg_table: recursion differs from the closed form at L = 3\n");
        return 1;
      }
    }
    bank(0.0, 0.0, 1.0, Y);
    for (int L = 2; L <= SL; ++L)
      if (std::abs(Y[L][L] - std::sqrt(2.0 * L + 1)) > 1e-5) {
        std::fprintf(stderr, "gen_cg_table: z-axis check failed at L = %d\n", L);
        return 1;
      }
  }
  std::fprintf(f, "inline constexpr int kShLmax = %d;\n", SL);
  std::fprintf(f, "inline constexpr int kShRecOff[%d] = {", SL + 1);
  for (int L = 0; L <= SL; ++L) std::fprintf(f, "%d%s", soff[L], L < SL ? ", " : "};\n");
  std::fprintf(f, "inline constexpr int kShRecCnt[%d] = {", SL + 1);
  for (int L = 0; L <= SL; ++L) std::fprintf(f, "%d%s", scnt[L], L < SL ? ", " : "};\n");
  std::fprintf(f, "inline constexpr float kShInvKappa[%d] = {", SL + 1);
  for (int L = 0; L <= SL; ++L)
    std::fprintf(f, "%a%s", double(float(inv_kappa[L])), L < SL ? ", " : "};\n");
  std::fprintf(f, "inline constexpr CgRec kShRec[%zu] = {\n", srec.size());
  for (const R& r : srec) std::fprintf(f, "  {%d, %d, %d, %a},\n", r.M, r.m1, r.m2, double(r.c));
  std::fprintf(f, "};\n\n");
  // the same recursion with coefficients kept in double, for the harmonics
  // evaluated in fp64 and rounded once
  std::fprintf(f, "struct CgRecD {\n  int M, m1, m2;\n  double c;\n};\n\n");
  std::fprintf(f, "inline constexpr double kShInvKappaD[%d] = {", SL + 1);
  for (int L = 0; L <= SL; ++L) std::fprintf(f, "%a%s", inv_kappa[L], L < SL ? ", " : "};\n");
  std::fprintf(f, "inline constexpr CgRecD kShRecD[%zu] = {\n", srec.size());
  for (const R& r : srec) std::fprintf(f, "  {%d, %d, %d, %a},\n", r.M, r.m1, r.m2, r.cd);
  std::fprintf(f, "};\n\n}  // namespace e3k\n");
  std::fclose(f);
  return 0;
}
