// CPU check of the row-split dK/dV map (moda_bwd_split.hpp), compiled with the
// host compiler alone: for many shapes, the closed forms the kernels use must
// agree with plain loops over the key tiles, every query block of every tile
// must be swept by exactly one chunk, chunk slots must be distinct and inside
// the workspace the plan sizes, and the remainder chunks must come longest
// first.  Prints "ok" and returns 0, or names the first failure and returns 1.
#define MODA_HD
#include "moda_bwd_split.hpp"

#include <cstdio>
#include <vector>

using moda::BwdChunkMap;

static int fail(const char* what, int T, int G, long long BH, int x) {
  std::printf("FAIL %s T=%d G=%d BH=%lld at %d\n", what, T, G, BH, x);
  return 1;
}

static int check(int T, int G, long long BH) {
  const int nkt = (T + 127) / 128;
  const moda::BwdSplitPlan pl = moda::bwd_split_plan(T, G, BH, nkt, 256);
  if (pl.C == 0) return 0;
  if (pl.C % (2 * G) != 0) return fail("C not a multiple of 2G", T, G, BH, pl.C);
  const BwdChunkMap cm(T, G, pl.C, nkt);
  const long long NQ = ((long long)T * G + 63) / 64;
  // closed forms against loops
  int pre = 0;
  for (int k = 0; k < nkt; ++k) {
    const long long n = NQ - 2LL * G * k;   // blocks of tile k: rows from 128 G k to T G
    if (cm.nqb(k) != n) return fail("nqb", T, G, BH, k);
    if (cm.nf(k) != n / pl.C || cm.rem(k) != n % pl.C) return fail("nf/rem", T, G, BH, k);
    if (cm.prefix(k) != pre) return fail("prefix", T, G, BH, k);
    pre += (int)(n / pl.C);
  }
  if (cm.prefix(nkt) != pre || pre != pl.full) return fail("full count", T, G, BH, pre);
  // walk the items as the dK/dV kernel does
  std::vector<std::vector<int>> cover(nkt);
  for (int k = 0; k < nkt; ++k) cover[k].assign(cm.nqb(k), 0);
  std::vector<int> slot_tile(pl.items, -1);
  int prev_rem = 1 << 30;
  for (int item = 0; item < pl.items; ++item) {
    int kt, lo, hi;
    if (item < pl.full) {
      kt = cm.full_tile(item);
      lo = (item - cm.prefix(kt)) * pl.C;
      hi = lo + pl.C;
    } else {
      kt = cm.rem_tile(item - pl.full);
      if (kt < 0 || kt >= nkt) return fail("rem_tile out of range", T, G, BH, item);
      lo = cm.nf(kt) * pl.C;
      hi = cm.nqb(kt);
      if (hi - lo > prev_rem) return fail("remainders not longest first", T, G, BH, item);
      prev_rem = hi - lo;
      if (cm.rem_rank(kt) != item - pl.full) return fail("rem_rank", T, G, BH, item);
    }
    if (kt < 0 || kt >= nkt || lo < 0 || hi > cm.nqb(kt) || lo >= hi) return fail("range", T, G, BH, item);
    for (int q = lo; q < hi; ++q) cover[kt][q]++;
    slot_tile[item] = kt;
  }
  if (cm.rem_tile(pl.items - pl.full) != -1) return fail("rem_tile past the end", T, G, BH, pl.items);
  for (int k = 0; k < nkt; ++k)
    for (int q = 0; q < cm.nqb(k); ++q)
      if (cover[k][q] != 1) return fail("block not swept exactly once", T, G, BH, k);
  // the reduce kernel's slots of tile kt are the items the kernel gave it
  for (int k = 0; k < nkt; ++k) {
    int n = 0;
    for (int c = 0; c < cm.nf(k); ++c) {
      const int it = cm.prefix(k) + c;
      if (it >= pl.items || slot_tile[it] != k) return fail("reduce full slot", T, G, BH, k);
      ++n;
    }
    if (cm.rem(k) > 0) {
      const int it = pl.full + cm.rem_rank(k);
      if (it >= pl.items || slot_tile[it] != k) return fail("reduce remainder slot", T, G, BH, k);
      ++n;
    }
    if (n != cm.nchunks(k)) return fail("nchunks", T, G, BH, k);
  }
  if ((long long)pl.items * BH > 256 + BH * nkt) return fail("chunk bound", T, G, BH, pl.items);
  return 1 << 16;   // split checked
}

int main() {
  int split = 0;
  const int Gs[] = {1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 32, 64};
  const long long BHs[] = {1, 2, 3, 4, 6, 8, 16, 32};
  for (int T = 1; T <= 20000; T += (T < 300 ? 1 : 97))
    for (int G : Gs)
      for (long long BH : BHs) {
        const int r = check(T, G, BH);
        if (r == 1) return 1;
        if (r) ++split;
      }
  const int big[][3] = {{65536, 8, 2}, {65536, 16, 1}, {32768, 8, 1}, {4096, 8, 2}, {16384, 8, 4}, {100000, 1, 1}};
  for (const auto& s : big) {
    const int r = check(s[0], s[1], s[2]);
    if (r == 1) return 1;
    if (r) ++split;
  }
  std::printf("ok (%d split shapes checked)\n", split);
  return 0;
}
