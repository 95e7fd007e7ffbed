// Placement of attention work items on the XCDs of an MI355X.
//
// A launch's work items are (head, block) pairs: B*H heads times `levels`
// blocks per head.  Workgroup g of a launch runs on XCD g % 8 (the hardware
// dispatches workgroups to the eight XCDs round-robin), and each XCD has its
// own L2.  Blocks of one head read the same K/V (forward, dQ) or Q/dO (dK/dV)
// tiles, so this placement keeps a head on as few XCDs as the work balance
// allows:
//   - with BH = 8a + b heads, XCD x gets the a whole heads x, x+8, ..,
//     x+8(a-1);
//   - the b remaining heads are cut into p residue classes of the block level
//     (level % p), p = 8 / gcd(b, 8), and XCD x gets c = b*p/8 consecutive
//     parts of them;
//   - an XCD runs its items heaviest first (level levels-1 down to 0), and at
//     each level its whole heads before its parts with that level's residue.
// Every XCD then holds BH*levels/8 items whose causal work differs only by the
// residue-class split.  The placement needs levels % p == 0 and is used only
// then; otherwise the launch keeps the plain order (level-major, heads
// fastest).  The arithmetic is host-and-device so that the host can verify it
// is a bijection before any launch relies on it.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct Placement {
  int BH, levels;   // heads and block levels per head
  int a, b, p, c;   // whole heads per XCD; leftover heads; parts per leftover head; parts per XCD
  int period;       // items per p consecutive levels on one XCD: a*p + c
  bool on;          // XCD-affine placement in use
};

__host__ __device__ inline int gcd_int(int x, int y) {
  while (y != 0) {
    const int t = x % y;
    x = y;
    y = t;
  }
  return x;
}

__host__ __device__ inline Placement make_placement(int BH, int levels) {
  Placement P{BH, levels, BH / 8, BH % 8, 1, 0, 0, false};
  P.p = P.b == 0 ? 1 : 8 / gcd_int(P.b, 8);
  P.c = P.b * P.p / 8;
  P.period = P.a * P.p + P.c;
  P.on = BH > 0 && levels > 0 && levels % P.p == 0;
  return P;
}

// Work item j (0-based) of XCD x: head `bh` and block level `level`
// (levels-1 is the first one the XCD runs).  Only valid when P.on and
// j < BH*levels/8.
__host__ __device__ inline void place_item(const Placement& P, int x, int j, int& bh, int& level) {
  const int pi = j / P.period;
  int o = j % P.period;
  const int k_begin = x * P.c;  // this XCD's parts: global part indices [k_begin, k_begin + c)
  for (int i = 0; i < P.p; ++i) {
    const int lev = P.levels - 1 - pi * P.p - i;
    if (o < P.a) {
      bh = x + 8 * o;
      level = lev;
      return;
    }
    o -= P.a;
    const int rho = lev % P.p;
    // parts k of this XCD with k % p == rho: k0, k0 + p, ...
    const int k0 = k_begin + ((rho - k_begin % P.p) + P.p) % P.p;
    const int n = k0 < k_begin + P.c ? (k_begin + P.c - 1 - k0) / P.p + 1 : 0;
    if (o < n) {
      const int k = k0 + o * P.p;
      bh = 8 * P.a + k / P.p;
      level = lev;
      return;
    }
    o -= n;
  }
  bh = -1;  // unreachable for valid (x, j): the p levels of a period hold exactly `period` items
  level = -1;
}

// Item of workgroup g in a launch of BH*levels workgroups: XCD-affine when
// P.on, else level-major with heads fastest.  `pair_stride` > 0 reverses
// every other group of that many items within an XCD, so that when
// workgroups g and g + 8*pair_stride share a compute unit, heavy and light
// items pair up there.
__host__ __device__ inline void place_workgroup(const Placement& P, int g, int pair_stride, int& bh, int& level) {
  if (!P.on) {
    if (pair_stride > 0) {
      const int G = 8 * pair_stride, total = P.BH * P.levels;
      const int grp = g / G, t = g % G;
      if ((grp & 1) && (grp + 1) * G <= total) g = grp * G + (G - 1 - t);
    }
    bh = g % P.BH;
    level = P.levels - 1 - g / P.BH;
    return;
  }
  const int x = g & 7;
  int j = g >> 3;
  if (pair_stride > 0) {
    const int per_xcd = P.BH * P.levels / 8;
    const int grp = j / pair_stride, t = j % pair_stride;
    if ((grp & 1) && (grp + 1) * pair_stride <= per_xcd) j = grp * pair_stride + (pair_stride - 1 - t);
  }
  place_item(P, x, j, bh, level);
}

}  // namespace fa
