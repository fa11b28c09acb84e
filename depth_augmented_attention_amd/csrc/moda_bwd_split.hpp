// Row-split dK/dV for short sequences: the plan and the index map shared by
// the host (workspace size, grid) and the device (which rows a workgroup
// sweeps, where its partial sums go).
//
// The dK/dV kernel gives each key tile of 128 keys (per batch and kv head)
// one workgroup, which sweeps every query row that can see those keys: under
// the causal mask (mhpn.cn article "动态混合深度注意力机制MoDA技术解析",
// section 2.2) the first tile meets all T * G rows and the last only its own.
// When the grid is small the first tiles alone set the run time.  Here each
// tile's query blocks (64 rows) are cut into chunks of C blocks, C a multiple
// of 2G; chunk c of tile kt sweeps blocks [c C, c C + C) of the tile's sweep
// order (block 0 holds the last rows), the remainder chunk the blocks left
// over (the ones on the diagonal).  Workgroups take, in blockIdx order, first
// every full chunk (key tile by key tile), then the remainder chunks from the
// longest to the shortest, so that the greedy dispatch of workgroups to
// compute units runs the long ones first.  A tile with more than one chunk
// writes float32 partial sums that a second kernel adds up in chunk order
// (full chunks, then the remainder): the result does not depend on timing.
//
// Tile kt has nqb(kt) = NQ - 2 G kt query blocks, NQ = ceil(T G / 64): its
// first row is 128 G kt, a multiple of 64.  Writing NQ = 2 G a + b
// (0 <= b < 2 G) and C = 2 G m:
//   full chunks  nf(kt) = floor((a - kt) / m)
//   remainder    r(kt)  = 2 G ((a - kt) mod m) + b   (no remainder chunk if 0)
// so the remainders fall in m classes u = (a - kt) mod m, larger u meaning a
// longer remainder, and the full chunks before tile kt number
//   prefix(kt) = S(a) - S(a - kt),  S(n) = sum_{j=0..n} floor(j / m).
#pragma once

#ifndef MODA_HD
#define MODA_HD __host__ __device__
#endif

namespace moda {

struct BwdChunkMap {
  int G, C, m, a, b, nkt;

  MODA_HD BwdChunkMap(int T, int G_, int C_, int nkt_) : G(G_), C(C_), m(C_ / (2 * G_)), nkt(nkt_) {
    const long long nq = ((long long)T * G_ + 63) / 64;
    a = (int)(nq / (2 * G_));
    b = (int)(nq % (2 * G_));
  }
  MODA_HD int nqb(int kt) const { return 2 * G * (a - kt) + b; }
  MODA_HD int nf(int kt) const { return (a - kt) / m; }
  MODA_HD int rem(int kt) const { return 2 * G * ((a - kt) % m) + b; }
  MODA_HD int nchunks(int kt) const { return nf(kt) + (rem(kt) > 0 ? 1 : 0); }
  MODA_HD long long S(long long n) const {
    if (n < 0) return 0;
    const long long q = n / m, s = n % m;
    return m * q * (q - 1) / 2 + q * (s + 1);
  }
  // full chunks of tiles 0 .. kt-1
  MODA_HD int prefix(int kt) const { return (int)(S(a) - S(a - kt)); }
  // smallest tile of remainder class u, and the tiles of that class
  MODA_HD int k0(int u) const { return ((a - u) % m + m) % m; }
  MODA_HD int count(int u) const { return k0(u) < nkt ? (nkt - 1 - k0(u)) / m + 1 : 0; }
  MODA_HD int lowest_class() const { return b > 0 ? 0 : 1; }
  // tile of full chunk f (0 <= f < prefix(nkt)): the last kt with prefix(kt) <= f
  MODA_HD int full_tile(int f) const {
    int lo = 0, hi = nkt;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (prefix(mid) <= f) lo = mid; else hi = mid;
    }
    return lo;
  }
  // tile of the i-th remainder chunk (longest first, then by tile)
  MODA_HD int rem_tile(int i) const {
    for (int u = m - 1; u >= lowest_class(); --u) {
      const int c = count(u);
      if (i < c) return k0(u) + i * m;
      i -= c;
    }
    return -1;
  }
  // position of tile kt's remainder chunk among the remainder chunks
  MODA_HD int rem_rank(int kt) const {
    const int u = (a - kt) % m;
    int r = 0;
    for (int v = m - 1; v > u; --v) r += count(v);
    return r + (kt - k0(u)) / m;
  }
};

// The split chosen for a grid of BH = B * Hkv (batch, kv head) pairs over
// nkt key tiles, for a kernel running one workgroup per compute unit on
// `cus` compute units: C = the average work per compute unit (in query
// blocks, at least 16), rounded up to a multiple of 2 G; no split unless the
// first tile's sweep exceeds 1.25 C.  items = chunks per (b, kv head).
struct BwdSplitPlan {
  int C = 0, full = 0, items = 0;
};

inline BwdSplitPlan bwd_split_plan(int T, int G, long long BH, int nkt, int cus) {
  BwdSplitPlan pl;
  if (T < 1 || G < 1 || BH < 1 || nkt < 1 || nkt > 4096 || G > 1024) return pl;
  const long long NQ = ((long long)T * G + 63) / 64;
  long long W = 0;
  for (int k = 0; k < nkt; ++k) W += NQ - 2LL * G * k;
  W *= BH;
  long long C = (W + cus - 1) / cus;
  if (C < 16) C = 16;
  C = (C + 2 * G - 1) / (2 * G) * (2 * G);
  if (4 * NQ <= 5 * C) return pl;
  long long full = 0, rems = 0;
  for (int k = 0; k < nkt; ++k) {
    const long long n = NQ - 2LL * G * k;
    full += n / C;
    rems += n % C > 0;
  }
  pl.C = (int)C;
  pl.full = (int)full;
  pl.items = (int)(full + rems);
  return pl;
}

}  // namespace moda
