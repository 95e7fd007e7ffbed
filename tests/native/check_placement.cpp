// Host check of the XCD placement arithmetic (io_aware_exact_07_amd/csrc/fa_place.h):
// for every head count and block-level count in the ranges below, and with and
// without the CU-pairing reversal, every workgroup of a launch maps to a
// distinct (head, level) inside the launch's bounds, so the mapping is a
// bijection.  Also reports, for the XCD-affine cases, the largest number of
// distinct heads on one XCD and the spread of causal work (sum of level+1)
// across XCDs.  Prints "ok" and exits 0, or the first failure and exits 1.
#include <cstdio>
#include <vector>

#include "fa_place.h"

int main() {
  int checked = 0, affine = 0, worst_heads = 0;
  double worst_spread = 0.0;
  for (int BH = 1; BH <= 80; ++BH) {
    for (int levels = 1; levels <= 72; ++levels) {
      const fa::Placement P = fa::make_placement(BH, levels);
      for (int pair : {0, 32}) {
        std::vector<int> seen((size_t)BH * levels, 0);
        std::vector<long long> work(8, 0);
        std::vector<std::vector<int>> heads(8, std::vector<int>(BH, 0));
        for (int g = 0; g < BH * levels; ++g) {
          int bh = -1, lev = -1;
          fa::place_workgroup(P, g, pair, bh, lev);
          if (bh < 0 || bh >= BH || lev < 0 || lev >= levels) {
            std::printf("out of range: BH=%d levels=%d pair=%d g=%d -> (%d, %d)\n", BH, levels, pair, g, bh, lev);
            return 1;
          }
          if (seen[(size_t)bh * levels + lev]++) {
            std::printf("duplicate: BH=%d levels=%d pair=%d g=%d -> (%d, %d)\n", BH, levels, pair, g, bh, lev);
            return 1;
          }
          work[g & 7] += lev + 1;
          heads[g & 7][bh] = 1;
        }
        ++checked;
        if (P.on && pair == 0 && BH * levels >= 64) {
          ++affine;
          long long lo = work[0], hi = work[0];
          for (int x = 0; x < 8; ++x) {
            lo = work[x] < lo ? work[x] : lo;
            hi = work[x] > hi ? work[x] : hi;
            int n = 0;
            for (int h = 0; h < BH; ++h) n += heads[x][h];
            worst_heads = n > worst_heads ? n : worst_heads;
          }
          const double spread = (double)(hi - lo) / (double)hi;
          worst_spread = spread > worst_spread ? spread : worst_spread;
        }
      }
    }
  }
  std::printf("ok: %d launches checked, %d XCD-affine; causal work spread across XCDs at most %.3f\n", checked,
              affine, worst_spread);
  const fa::Placement P = fa::make_placement(12, 64);
  std::printf("12 heads x 64 levels: on=%d a=%d b=%d p=%d c=%d\n", (int)P.on, P.a, P.b, P.p, P.c);
  return 0;
}
