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

// First rows of every tile load (attn_common.hpp, "tile loads"): the direct
// global -> LDS load addresses a tile from its first row, which must be one
// of the tensor's rows.
static int imin_(int a, int b) { return a < b ? a : b; }

// General kernels: a workgroup owns rows [a, a + BM) of one tensor (query rows
// when by_query, else keys) and walks the visible range of the other in T-row
// tiles from range_tile_row(lo, T, 0) while the tile's first row is below hi.
static void check_range_loads(const MaskGeom& g, bool by_query, int BM, int T, const char* kernel) {
  const int n_own = by_query ? g.nq : g.nk;
  const int n_load = by_query ? g.nk : g.nq;
  for (int a = 0; a < n_own; a += BM) {
    const int b = imin_(a + BM, n_own);
    int lo, hi;
    if (by_query)
      g.key_range(a, b, &lo, &hi);
    else
      g.query_range(a, b, &lo, &hi);
    if (lo >= hi) continue;
    CHECK(lo >= 0 && hi <= n_load, "%s range [%d,%d) outside %d rows (m%d W%d %dx%d)\n", kernel, lo, hi, n_load,
          g.mode, g.window, g.nq, g.nk);
    for (int t = 0;; ++t) {
      const int r0 = attn::range_tile_row(lo, T, t);
      if (r0 >= hi) break;
      CHECK(r0 >= 0 && r0 < n_load, "%s tile row %d of %d rows (m%d W%d %dx%d, wg rows %d)\n", kernel, r0, n_load,
            g.mode, g.window, g.nq, g.nk, a);
    }
  }
}

static void check_general_loads(const MaskGeom& g) {
  check_range_loads(g, true, 128, 64, "fwd");          // 128 query rows, 64-key K/V tiles
  check_range_loads(g, false, 128, 64, "dkdv d<=96");  // 128 keys, 64-row Q/dO tiles
  check_range_loads(g, false, 128, 32, "dkdv d=128");  // 128 keys, 32-row Q/dO tiles
  check_range_loads(g, true, 128, 128, "dq kept dS");  // 128 query rows, 128-key K tiles
  check_range_loads(g, true, 128, 64, "dq");           // 128 query rows, 64-key K/V tiles
}

// The short-sequence backward, for every (Nq, Nk) and mask it accepts: key
// blocks (K from short_k_block_row, V from 32 b for the real blocks) and
// 32-row query slabs.
static long short_geometries = 0;
static void check_short_loads(const MaskGeom& g) {
  for (int d : {64, 96}) {
    if (!attn::short_keys(g, d)) continue;
    ++short_geometries;
    const int nkb = attn::short_key_blocks(g.nk);
    CHECK(nkb >= 1 && nkb <= attn::kShortKeys / 32, "short: %d key blocks for nk %d\n", nkb, g.nk);
    for (int b = 0; b < attn::kShortKeys / 32; ++b) {
      const int r0 = attn::short_k_block_row(b, g.nk);
      CHECK(r0 >= 0 && r0 < g.nk, "short: K block %d at row %d of %d (nq %d m%d d%d)\n", b, r0, g.nk, g.nq,
            g.mode, d);
      if (b < nkb) CHECK(32 * b < g.nk, "short: V block %d of %d keys\n", b, g.nk);
    }
    for (int s = 0; 32 * s < g.nq; ++s) CHECK(32 * s < g.nq, "short: slab %d of %d rows\n", s, g.nq);
  }
}

// Single-tile block-local kernels: tile t < ceil(nk / 64) of every local64()
// geometry starts inside both tensors and has at least one real query row.
static void check_local_loads(const MaskGeom& g) {
  if (!g.local64()) return;
  int lw = 0, lq = 0;
  while ((1 << lw) < g.window) ++lw;
  while ((1 << lq) < g.window_q) ++lq;
  for (int t = 0; 64 * t < g.nk; ++t) {
    const attn::LocalTile lt = attn::local_tile(t, g.nq, lw, lq);
    CHECK(lt.tk0 < g.nk && lt.tq0 < g.nq && lt.qend > lt.tq0 && lt.qend - lt.tq0 <= lt.qt,
          "local tile %d: keys from %d of %d, rows [%d,%d) of %d (W%d Wq%d)\n", t, lt.tk0, g.nk, lt.tq0, lt.qend,
          g.nq, g.window, g.window_q);
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
  // tile loads of the general kernels over a wider range of sizes
  const int lsizes[] = {1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 256, 257, 700};
  for (int nq : lsizes)
    for (int nk : lsizes) {
      check_general_loads(MaskGeom{attn::kNone, nq, nk, 0, 0});
      check_general_loads(MaskGeom{attn::kCausal, nq, nk, 0, 0});
      for (int W : {1, 2, 31, 64, 100, 1024}) check_general_loads(MaskGeom{attn::kSliding, nq, nk, W, 0});
      for (int W = 1; W <= nk; ++W)
        if (nk % W == 0 && nq % (nk / W) == 0) {
          const MaskGeom g{attn::kBlock, nq, nk, W, nq / (nk / W)};
          check_general_loads(g);
          check_local_loads(g);
        }
    }
  // the short-sequence backward: every Nk <= 224 and Nq <= 1024 under every mask
  for (int nk = 1; nk <= attn::kShortKeys; ++nk)
    for (int nq = 1; nq <= attn::kShortRows; ++nq) {
      check_short_loads(MaskGeom{attn::kNone, nq, nk, 0, 0});
      check_short_loads(MaskGeom{attn::kCausal, nq, nk, 0, 0});
      for (int W : {1, 7, 64, 200, 1000}) check_short_loads(MaskGeom{attn::kSliding, nq, nk, W, 0});
      for (int W = 1; W <= nk; ++W)
        if (nk % W == 0 && nq % (nk / W) == 0) check_short_loads(MaskGeom{attn::kBlock, nq, nk, W, nq / (nk / W)});
    }
  CHECK(short_geometries > 1000000, "short: only %ld geometries checked\n", short_geometries);
  // the check above would have caught K blocks loaded from row 32 b: that
  // first row is past the keys for every nk <= kShortKeys - 32
  int unclamped_bad = 0;
  for (int nk = 1; nk <= attn::kShortKeys; ++nk)
    for (int b = 0; b < attn::kShortKeys / 32; ++b) unclamped_bad += 32 * b >= nk;
  CHECK(unclamped_bad > 0, "the unclamped K block rows were never out of range\n");
  std::printf("%ld short-backward geometries\n", short_geometries);
  std::printf("%d failures\n", fails);
  return fails ? 1 : 0;
}
