// attn_common.hpp -- shared definitions of the gfx950 attention kernels:
// launch parameters, the per-row / per-key visibility intervals that drive
// tile ranges and masking, and thin wrappers over the CDNA4 MFMA and LDS
// transpose-read builtins.
//
// Visibility (all four mask modes) is an interval per query row i:
//     key j is visible to i  <=>  row_lo(i) <= j < row_hi(i)
//   none    [0, Nk)
//   causal  [0, min(i + 1, Nk))
//   sliding [max(0, i - W + 1), min(i + 1, Nk))     W keys incl. the diagonal
//                                                   ("IHA-CUDA", FLOP Matching)
//   block   [floor(i/Wq)*W, floor(i/Wq)*W + W)          independent windows
//                                                   of W keys and Wq query
//                                                   rows ("hiera-optim" sdist,
//                                                   MaskUnitAttentionFast;
//                                                   Wq < W with pooled queries)
// and, equivalently, an interval of queries per key j:
//     col_lo(j) <= i < col_hi(j).
// Both bounds are non-decreasing in i (resp. j), so the keys a block of rows
// [a, b) can see are [row_lo(a), row_hi(b-1)), and a rows x keys tile is fully
// visible iff its keys lie in [row_lo(b-1), row_hi(a)).  This is the tile-range
// computation ("IHA-CUDA", Repository Structure: block_info / mask) written as
// intervals.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define ATTN_HD __host__ __device__ __forceinline__
#else
#define ATTN_HD inline
#endif

namespace attn {

enum MaskMode : int { kNone = 0, kCausal = 1, kSliding = 2, kBlock = 3 };
// kernel template argument: the mask mode is read from MaskGeom at run time
constexpr int kAnyMask = -1;

struct MaskGeom {
  int mode;
  int nq, nk;
  int window;    // W for sliding, the key window length for block; unused otherwise
  int window_q;  // block: query rows per window (= window unless queries are pooled)

  ATTN_HD int imin(int a, int b) const { return a < b ? a : b; }
  ATTN_HD int imax(int a, int b) const { return a > b ? a : b; }

  // keys visible to query row i: [row_lo(i), row_hi(i))
  ATTN_HD int row_lo(int i) const {
    if (mode == kSliding) return imax(0, i - window + 1);
    if (mode == kBlock) return (i / window_q) * window;
    return 0;
  }
  ATTN_HD int row_hi(int i) const {
    if (mode == kCausal || mode == kSliding) return imin(i + 1, nk);
    if (mode == kBlock) return imin((i / window_q) * window + window, nk);
    return nk;
  }
  // queries that see key j: [col_lo(j), col_hi(j))
  ATTN_HD int col_lo(int j) const {
    if (j >= nk) return nq;
    if (mode == kCausal || mode == kSliding) return imin(j, nq);
    if (mode == kBlock) return imin((j / window) * window_q, nq);
    return 0;
  }
  ATTN_HD int col_hi(int j) const {
    if (j >= nk) return nq;
    if (mode == kSliding) return imin(j + window, nq);
    if (mode == kBlock) return imin((j / window) * window_q + window_q, nq);
    return nq;
  }
  // keys visible to any row of [a, b) (b > a): [lo, hi), possibly empty
  ATTN_HD void key_range(int a, int b, int* lo, int* hi) const {
    *lo = row_lo(a);
    *hi = row_hi(b - 1);
  }
  // queries that see any key of [a, b) (b > a)
  ATTN_HD void query_range(int a, int b, int* lo, int* hi) const {
    *lo = col_lo(a);
    *hi = col_hi(imin(b, nk) - 1);
    if (a >= nk) *hi = *lo;
  }
  // every query row sees only keys of its own 64-key tile: block-local with a
  // key window dividing 64 and a query window dividing the key window (both
  // then powers of two); tile t holds keys [64 t, 64 t + 64) and query rows
  // [QT t, QT t + QT), QT = 64 / window * window_q
  ATTN_HD bool local64() const {
    return mode == kBlock && window >= 1 && 64 % window == 0 && window_q >= 1 &&
           window % window_q == 0;
  }
  // every (row, key) of rows [a, b) x keys [j0, j1) visible; needs b <= nq, j1 <= nk
  ATTN_HD bool tile_full(int a, int b, int j0, int j1) const {
    if (b > nq || j1 > nk) return false;
    return j0 >= row_lo(b - 1) && j1 <= row_hi(a);
  }

  // dS blocks kept by the backward for its dQ pass: one 32 x 32 block per
  // (key block kb = keys 32 kb .. 32 kb + 31, query block jb = rows 32 jb ..
  // 32 jb + 31) pair that has a visible entry.  The query blocks of key block
  // kb that do are the contiguous range [ds_jlo(kb), ds_jlo(kb) + ds_count(kb)).
  ATTN_HD void ds_rows(int kb, int* lo, int* hi) const {
    const int a = 32 * kb;
    if (a >= nk) {
      *lo = *hi = 0;
      return;
    }
    query_range(a, imin(a + 32, nk), lo, hi);
  }
  ATTN_HD int ds_jlo(int kb) const {
    int lo, hi;
    ds_rows(kb, &lo, &hi);
    return lo / 32;
  }
  ATTN_HD int ds_count(int kb) const {
    int lo, hi;
    ds_rows(kb, &lo, &hi);
    return lo < hi ? (hi + 31) / 32 - lo / 32 : 0;
  }
  // blocks per (b, h): the sum of ds_count over the key blocks
  ATTN_HD int64_t ds_blocks() const {
    int64_t n = 0;
    for (int kb = 0; 32 * kb < nk; ++kb) n += ds_count(kb);
    return n;
  }
};

// The fused backward for short key sequences holds every key of a (b, h) in
// one workgroup: one wave per 32 keys and a dQ wave, 8 waves at most.  It
// loops over the query rows in slabs of 32, so long query sequences are left
// to the general passes.
constexpr int kShortKeys = 224;
constexpr int kShortRows = 1024;
inline bool short_keys(const MaskGeom& g, int d) {
  return !g.local64() && (d == 64 || d == 96) && g.nk <= kShortKeys && g.nq <= kShortRows;
}

// elements of one dS block: 2 key chunks x 64 lanes x 8 bf16
constexpr int kDsBlockElems = 1024;

// ---------------------------------------------------------------- tile loads

// Every kernel moves rows a tile at a time.  The direct global -> LDS tile
// load addresses a tile of contiguous rows from its first row r0, so r0 must
// lie inside the tensor's n rows (rows past n inside the tile read row n - 1).
// The first rows of all tile loads come from the functions below, which
// tests/host/tile_range_check.cpp enumerates on the host for every geometry
// the kernels accept, checking r0 < n.

// A loop over the visible range [lo, hi) (lo < hi <= n) in T-row tiles aligned
// to multiples of T: tile t starts at range_tile_row(lo, T, t) and is loaded
// only while that row is below hi.
ATTN_HD int range_tile_row(int lo, int T, int t) { return (lo / T) * T + t * T; }

// The short-sequence backward's key blocks of 32 rows: nk keys fill
// short_key_blocks(nk) blocks.  Its unrolled loops run over all
// kShortKeys / 32 blocks; block b's K rows are loaded from row
// short_k_block_row(b, nk), which repeats the last real block for the blocks
// past the keys (finite values whose dS and partial row sums stay zero).
// Loading block b from row 32 b would address rows past the slice for the
// blocks past the keys, i.e. whenever nk <= kShortKeys - 32.
ATTN_HD int short_key_blocks(int nk) { return (nk + 31) / 32; }
ATTN_HD int short_k_block_row(int b, int nk) {
  const int last = short_key_blocks(nk) - 1;
  return 32 * (b < last ? b : last);
}

// Single-tile block-local geometry (MaskGeom::local64): key window w = 1 << lw,
// query rows per window wq = 1 << lq; tile t holds keys [64 t, 64 t + 64) and
// query rows [QT t, QT t + QT) with QT = (64 >> lw) << lq, of which the rows
// below qend are real.  For t < ceil(nk / 64) both first rows are inside
// their tensors: 64 t < nk, and QT t < nq since nq = (nk >> lw) << lq.
struct LocalTile {
  int lw, lq, qt;  // log2 w, log2 wq, query rows per tile
  int tk0;         // first key of the tile
  int tq0, qend;   // first query row of the tile, end of its real rows
  ATTN_HD bool real(int r) const { return tq0 + r < qend; }  // implies r < qt
  // bitwise, not short-circuit: evaluated per score element without branches
  ATTN_HD bool vis(int r, int c) const { return real(r) & ((r >> lq) == (c >> lw)); }
};
ATTN_HD LocalTile local_tile(int tile, int nq, int lw, int lq) {
  LocalTile t;
  t.lw = lw;
  t.lq = lq;
  t.qt = (64 >> lw) << lq;
  t.tk0 = tile * 64;
  t.tq0 = tile * t.qt;
  t.qend = t.tq0 + t.qt < nq ? t.tq0 + t.qt : nq;
  return t;
}

// ---------------------------------------------------------------- row maps

// Where the rows of one [B][H][N][d] tensor live.  Row j (token j) of slice
// (b, h) starts at element
//     b * batch + h * head + (j >> wshift) * win + (j & wmask) * tok
// of the tensor's base pointer, and its d values are contiguous.  A tensor
// in one window per slice (every contiguous layout, and any strided one whose
// windows follow each other at a uniform token stride) has wshift = 31,
// wmask = 0x7fffffff, win = 0.  The host guarantees that the in-slice offset
// of every row fits in 31 bits.
struct RowMap {
  int64_t batch, head;
  int32_t win, tok;
  int32_t wshift, wmask;

  // element offset of slice bh = b * H + h
  ATTN_HD int64_t slice(int bh, int H) const {
    return (int64_t)(bh / H) * batch + (int64_t)(bh % H) * head;
  }
  // element offset of row j inside its slice
  ATTN_HD uint32_t row(int j) const {
    return (uint32_t)(j >> wshift) * (uint32_t)win + (uint32_t)(j & wmask) * (uint32_t)tok;
  }
  // the contiguous layout of an [H][n][d] slice set: row j at j * d
  ATTN_HD bool plain(int H, int n, int d) const {
    return wshift == 31 && tok == d && batch == (int64_t)H * n * d && head == (int64_t)n * d;
  }
};

// Row addressing for kernels compiled per layout class: SR = false is the
// contiguous layout (slice bh at bh * n * D, row j at j * D, both folded at
// compile time), SR = true reads the RowMap.
template <bool SR, int D>
ATTN_HD uint32_t rrow(const RowMap& m, int j) {
  if constexpr (SR) return m.row(j);
  else return (uint32_t)j * D;
}
template <bool SR, int D>
ATTN_HD int64_t rslice(const RowMap& m, int bh, int H, int n) {
  if constexpr (SR) return m.slice(bh, H);
  else return (int64_t)bh * n * D;
}

// ---------------------------------------------------------------- launches

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // [B][H][Nq], contiguous
  RowMap rq, rk, rv, ro;
  int B, H, nq, nk;
  float scale;
  MaskGeom mg;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  RowMap rq, rk, rv, ro, rdo, rdq, rdk, rdv;
  float* dsum;  // workspace: D_i = sum_c dO[i][c] * O[i][c], fp32 [B][H][Nq]
  // optional workspace part: dS blocks written by the dK/dV pass and read by
  // the dQ pass instead of recomputing S and dP (null: recompute);
  // ds_per_bh = MaskGeom::ds_blocks() blocks per (b, h)
  uint16_t* ds;
  int64_t ds_per_bh;
  int B, H, nq, nk;
  float scale;
  MaskGeom mg;
};

// IHA premix (pseudo-token construction) and its backward.  x, dx
// [B][N][H][d]; w [H][P][H] (input type); out, dout [B][H][N][P][d]; dw
// [H][P][H] fp32; dw_part: `grid` partial dW blocks of H*P*H fp32.
struct PremixArgs {
  const void* x;
  const void* w;
  void* out;
  const void* dout;
  void* dx;
  float* dw;
  float* dw_part;
  int B, N, H, lp;  // lp = log2(P)
  int grid;         // workgroups; also the number of dW partials
};

// every tensor of a call in the contiguous layout (the SR = false kernels)
inline bool rows_plain(const FwdArgs& a, int d) {
  return a.rq.plain(a.H, a.nq, d) && a.rk.plain(a.H, a.nk, d) && a.rv.plain(a.H, a.nk, d) &&
         a.ro.plain(a.H, a.nq, d);
}
inline bool rows_plain(const BwdArgs& a, int d) {
  return a.rq.plain(a.H, a.nq, d) && a.rk.plain(a.H, a.nk, d) && a.rv.plain(a.H, a.nk, d) &&
         a.ro.plain(a.H, a.nq, d) && a.rdo.plain(a.H, a.nq, d) && a.rdq.plain(a.H, a.nq, d) &&
         a.rdk.plain(a.H, a.nk, d) && a.rdv.plain(a.H, a.nk, d);
}

// The (b, h) slice and tile index of workgroup L of a BH x nt grid.  Tiles
// are taken heaviest first (`first_heavy`: query tile nt - 1 first when true,
// key tile 0 first when false; causal and sliding masks give the late query
// tiles / early key tiles the most work).  Under a causal mask the grid keeps
// one tile index across all slices at a time, for load balance.  Other masks
// lay the workgroups out XCD by XCD: the dispatcher sends workgroup L to XCD
// L % 8, and XCD x takes the contiguous run of (slice, tile) items starting
// at x q + min(x, r) (BH nt = 8 q + r), tiles of a slice adjacent, so tiles
// that read the same K/V (or Q/dO) rows run on one XCD and share its L2.
struct TileId {
  int bh, t;
};
ATTN_HD TileId tile_of(int L, int BH, int nt, bool causal, bool first_heavy) {
  if (causal) return {L % BH, first_heavy ? nt - 1 - L / BH : L / BH};
  const int x = L & 7, T = BH * nt, q = T >> 3, r = T & 7;
  const int item = x * q + (x < r ? x : r) + (L >> 3);
  const int t = item % nt;
  return {item / nt, first_heavy ? nt - 1 - t : t};
}

// backward pass bits (the values of include/attn.h's ATTN_PASS_*)
enum BwdPass : int { kPassRowSum = 1, kPassDKDV = 2, kPassDQ = 4, kPassAll = 7 };

}  // namespace attn

#if defined(__HIPCC__)
namespace attn {
// Launchers: the 16-bit ones (bf16, or fp16 with f16 set) and the fp32 ones;
// each picks its kernel instantiation from (d, mask, layout).  They return the
// hipError_t of the launch(es) as an int.  `passes` is a set of backward pass
// bits (row sums, dK/dV, dQ), launched in that order.
int launch_fwd_16(const FwdArgs& a, bool f16, int d, hipStream_t s);
int launch_bwd_16(const BwdArgs& a, bool f16, int d, hipStream_t s, int passes);
int launch_fwd_fp32(const FwdArgs& a, int d, hipStream_t s);
// single-tile 16-bit kernels for MaskGeom::local64() (forward; fused backward)
int launch_fwd_16_local(const FwdArgs& a, bool f16, int d, hipStream_t s);
int launch_bwd_16_local(const BwdArgs& a, bool f16, int d, hipStream_t s);
// fused 16-bit backward for short_keys() (one workgroup per (b, h))
int launch_bwd_16_short(const BwdArgs& a, bool f16, int d, hipStream_t s);
int launch_bwd_fp32(const BwdArgs& a, int d, hipStream_t s, int passes);
// IHA premix (16-bit types)
int launch_premix_fwd(const PremixArgs& a, bool f16, int d, hipStream_t s);
int launch_premix_bwd(const PremixArgs& a, bool f16, int d, hipStream_t s);
}  // namespace attn
#endif
