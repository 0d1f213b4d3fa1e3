// Brute-force check of the visibility intervals and tile predicates of
// attn_common.hpp (host build, no GPU).  Exit status 0 iff every check holds.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "attn_common.hpp"

using attn::MaskGeom;

static int g_wq = 0;  // block: query rows per window of the case being checked

static bool sees(int mode, int W, int nk, int i, int j) {
  if (j < 0 || j >= nk) return false;
  switch (mode) {
    case attn::kNone: return true;
    case attn::kCausal: return j <= i;
    case attn::kSliding: return i - W < j && j <= i;
    case attn::kBlock: return i / g_wq == j / W;
  }
  return false;
}

static int fails = 0;
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      if (fails < 20) std::printf(__VA_ARGS__);         \
      ++fails;                                          \
    }                                                   \
  } while (0)

static void check(int mode, int W, int nq, int nk) {
  g_wq = mode == attn::kBlock ? nq / (nk / W) : 0;
  MaskGeom g{mode, nq, nk, W, g_wq};
  for (int i = 0; i < nq; ++i)
    for (int j = 0; j < nk; ++j) {
      const bool v = sees(mode, W, nk, i, j);
      CHECK(v == (g.row_lo(i) <= j && j < g.row_hi(i)), "row interval m%d W%d %dx%d i%d j%d\n", mode, W,
            nq, nk, i, j);
      CHECK(v == (g.col_lo(j) <= i && i < g.col_hi(j)), "col interval m%d W%d %dx%d i%d j%d\n", mode, W,
            nq, nk, i, j);
    }
  // single-tile geometry of block-local shapes with local64(): tile t holds
  // keys [64 t, 64 t + 64) and query rows [QT t, QT t + QT); inside a tile,
  // row r and key c see each other iff r >> log2(Wq) == c >> log2(W)
  if (g.local64()) {
    int lw = 0, lq = 0;
    while ((1 << lw) < W) ++lw;
    while ((1 << lq) < g_wq) ++lq;
    CHECK((1 << lw) == W && (1 << lq) == g_wq, "local64 windows not powers of two W%d Wq%d\n", W, g_wq);
    const int qt = (64 >> lw) << lq;
    for (int i = 0; i < nq; ++i)
      for (int j = 0; j < nk; ++j) {
        const bool v = sees(mode, W, nk, i, j);
        if (v) CHECK(i / qt == j / 64, "local64 pair crosses tiles W%d %dx%d i%d j%d\n", W, nq, nk, i, j);
        if (i / qt == j / 64)
          CHECK(v == (((i % qt) >> lq) == ((j % 64) >> lw)), "local64 in-tile rule W%d %dx%d i%d j%d\n",
                W, nq, nk, i, j);
      }
  }
  const int steps[] = {1, 3, 4, 7, 16, 32};
  for (int bs : steps) {
    for (int a = 0; a < nq; a += bs) {
      const int b = a + bs < nq ? a + bs : nq;
      int lo, hi;
      g.key_range(a, b, &lo, &hi);
      for (int j = 0; j < nk; ++j) {
        bool any = false;
        for (int i = a; i < b; ++i) any |= sees(mode, W, nk, i, j);
        if (any) CHECK(lo <= j && j < hi, "key_range misses m%d W%d rows[%d,%d) j%d\n", mode, W, a, b, j);
      }
      // tight: the ends of a non-empty range are visible to some row
      if (lo < hi) {
        bool e0 = false, e1 = false;
        for (int i = a; i < b; ++i) {
          e0 |= sees(mode, W, nk, i, lo);
          e1 |= sees(mode, W, nk, i, hi - 1);
        }
        CHECK(e0 && e1, "key_range loose m%d W%d rows[%d,%d) [%d,%d)\n", mode, W, a, b, lo, hi);
      }
      for (int j0 = 0; j0 < nk; j0 += bs) {
        const int j1 = j0 + bs;
        bool all = b <= nq && j1 <= nk;
        for (int i = a; i < b && all; ++i)
          for (int j = j0; j < j1 && all; ++j) all = sees(mode, W, nk, i, j);
        CHECK(all == g.tile_full(a, b, j0, j1), "tile_full m%d W%d rows[%d,%d) keys[%d,%d)\n", mode, W,
              a, b, j0, j1);
      }
    }
    for (int a = 0; a < nk; a += bs) {
      const int b = a + bs;
      int lo, hi;
      g.query_range(a, b, &lo, &hi);
      for (int i = 0; i < nq; ++i) {
        bool any = false;
        for (int j = a; j < b && j < nk; ++j) any |= sees(mode, W, nk, i, j);
        if (any) CHECK(lo <= i && i < hi, "query_range misses m%d W%d keys[%d,%d) i%d\n", mode, W, a, b, i);
      }
      if (lo < hi) {
        bool e0 = false, e1 = false;
        for (int j = a; j < b && j < nk; ++j) {
          e0 |= sees(mode, W, nk, lo, j);
          e1 |= sees(mode, W, nk, hi - 1, j);
        }
        CHECK(e0 && e1, "query_range loose m%d W%d keys[%d,%d) [%d,%d)\n", mode, W, a, b, lo, hi);
      }
    }
  }
}

// workgroup -> (slice, tile) order of the general kernels: every (slice,
// tile) pair exactly once; causal grids keep one tile index across all
// slices at a time, heaviest first; other grids give each XCD (workgroup
// L -> XCD L % 8) one contiguous run of items, tiles of a slice adjacent
static void check_tile_order(int BH, int nt) {
  const int T = BH * nt;
  for (int causal = 0; causal < 2; ++causal)
    for (int heavy = 0; heavy < 2; ++heavy) {
      std::vector<int> seen(T, 0);
      for (int L = 0; L < T; ++L) {
        const attn::TileId t = attn::tile_of(L, BH, nt, causal, heavy);
        CHECK(t.bh >= 0 && t.bh < BH && t.t >= 0 && t.t < nt, "tile_of out of range BH%d nt%d L%d\n", BH, nt, L);
        if (t.bh >= 0 && t.bh < BH && t.t >= 0 && t.t < nt) ++seen[t.bh * nt + t.t];
        if (causal) {
          CHECK(t.bh == L % BH && t.t == (heavy ? nt - 1 - L / BH : L / BH), "causal order BH%d nt%d L%d\n", BH,
                nt, L);
        } else if (L >= 8) {
          // the previous workgroup of the same XCD took the preceding item
          const attn::TileId p = attn::tile_of(L - 8, BH, nt, causal, heavy);
          const int item = t.bh * nt + (heavy ? nt - 1 - t.t : t.t);
          const int prev = p.bh * nt + (heavy ? nt - 1 - p.t : p.t);
          CHECK(item == prev + 1, "XCD run not contiguous BH%d nt%d L%d\n", BH, nt, L);
        }
      }
      for (int e = 0; e < T; ++e) CHECK(seen[e] == 1, "tile_of not a bijection BH%d nt%d item%d\n", BH, nt, e);
    }
}

int main() {
  const int bhs[] = {1, 3, 8, 20, 80, 512};
  const int nts[] = {1, 2, 7, 32, 64};
  for (int bh : bhs)
    for (int nt : nts) check_tile_order(bh, nt);

  const int sizes[] = {1, 2, 4, 5, 16, 17, 33, 64, 65, 96, 128};
  for (int nq : sizes)
    for (int nk : sizes) {
      check(attn::kNone, 0, nq, nk);
      check(attn::kCausal, 0, nq, nk);
      const int wins[] = {1, 2, 3, 16, 40, 100};
      for (int W : wins) check(attn::kSliding, W, nq, nk);
      // block: nk / W windows of W keys, nq / (nk / W) query rows each
      // (nq < nk: pooled queries)
      for (int W = 1; W <= nk; ++W)
        if (nk % W == 0 && nq % (nk / W) == 0) check(attn::kBlock, W, nq, nk);
    }
  std::printf("%d failures\n", fails);
  return fails ? 1 : 0;
}
