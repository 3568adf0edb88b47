// Build step: writes the compile-time CG record table that the gfx950
// kernels unroll.  For every coupled triple (l1, l2, L) with l1, l2, L <= 3
// it lists the nonzero entries of the real block from cg_real_block(), as
// records (M, m1, m2, c) sorted by (M, m1, m2), with c rounded to fp32.
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
              recs.push_back({M, a, b, float(v)});
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
  std::fprintf(f, "};\n\n}  // namespace e3k\n");
  std::fclose(f);
  return 0;
}
