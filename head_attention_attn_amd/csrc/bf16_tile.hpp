// bf16_tile.hpp -- LDS tile layout and tile movement shared by the bf16
// attention kernels: direct global -> LDS tile loads, MFMA operand reads
// (row-wise and transposed), accumulator -> LDS staging and LDS -> global
// row stores.
//
// LDS tile layout.  A ROWS x D bf16 tile is stored row-major with row stride
// tstride<D>() elements; within row r the 16-byte chunk c (elements 8c ..
// 8c+7) sits at chunk position c ^ ((r / 4) % 4).  gfx950's LDS has 64
// four-byte banks and serves a ds_read_b128 16 lanes at a time and a
// ds_read_b64 / ds_read_b64_tr_b16 32 lanes at a time (measured with
// SQ_LDS_BANK_CONFLICT on MI355X).  The kernels read tiles in two patterns:
//   row reads   lanes 0..15 read the same chunk of 16 consecutive rows;
//   transposed  lanes 0..31 read 4 consecutive rows (a multiple of 4 first)
//               x 4 consecutive chunks (a multiple of 4 first).
// With a stride of 16 or 48 banks (mod 64) -- 160 elements for D = 128, 96 for
// D = 96 and D = 64 -- rows r .. r+3 start in four different 16-bank groups,
// which serves the transposed pattern; the row pattern's 16 rows then fall
// four to a group, and the XOR of the low two chunk bits with (r / 4) % 4
// spreads those four over the group's four 16-byte slots.  Both patterns run
// in one pass per 16 / 32 lanes.  The XOR touches only the low two chunk bits
// and depends on row bits 2-3 only, so most loop-varying offsets stay
// compile-time constants (ds_read immediate offsets) rather than per-lane
// address registers.
#pragma once

#include "attn_common.hpp"
#include "mfma.hpp"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

template <int D>
__host__ __device__ constexpr int tstride() {
  static_assert(D == 64 || D == 96 || D == 128, "head dim");
  return D == 128 ? 160 : 96;
}

// element offset of (row r, column col) in a tile; col % 4 == 0.  The
// 16-byte chunks of a row are permuted in groups of four by bits SW, SW + 1
// of the row: with SW = 2, 32 lanes reading rows 0..31 at one chunk are
// conflict-free; with SW = 1, 16 lanes reading rows 0..15 at one chunk (and
// the other 48 lanes the next chunks) are; the transposed reads are
// conflict-free under either
template <int D, int SW = 2>
__device__ __forceinline__ int toff(int r, int col) {
  return r * tstride<D>() + ((((col >> 3) ^ ((r >> SW) & 3)) << 3) | (col & 7));
}

// The same offset for row r0 + rl, column c0 + cl, written so that the part
// from r0 (a multiple of 16) and c0 (a multiple of 32) -- compile-time values
// in the kernels' unrolled loops -- is a plain sum: the swizzle then depends
// on the per-lane rl, cl only, and the compiler folds r0, c0 into the
// instruction's immediate offset.  0 <= cl < 32.
template <int D, int SW = 2>
__device__ __forceinline__ int toff2(int r0, int rl, int c0, int cl) {
  return (r0 + rl) * tstride<D>() + c0 + (((((cl >> 3) & 3) ^ ((rl >> SW) & 3)) << 3) | (cl & 7));
}

// elements of a ROWS-row tile
template <int ROWS, int D>
__host__ __device__ constexpr int tile_elems() {
  return ROWS * tstride<D>();
}

// MFMA operand from a row read: 8 consecutive bf16 of row r0 + rl at columns
// 16 kc + 8 gq .. +7 (the contraction runs along the row); r0 % 16 == 0.
template <int D, typename E>
__device__ __forceinline__ typename E::v8 lds_row8(const uint16_t* tile, int r0, int rl, int kc,
                                                   int gq) {
  return *reinterpret_cast<const typename E::v8*>(
      tile + toff2<D>(r0, rl, 32 * (kc >> 1), 16 * (kc & 1) + 8 * gq));
}

// Transposed operand read (ds_read_b64_tr_b16, see mfma.hpp): the 8
// contraction elements of an MFMA operand whose free index is the tile column
// c0 + lane % 32 and whose contraction runs over tile rows; slots 0..3 are
// rows r0 + 4g + e, slots 4..7 rows r0 + 8 + 4g + e (g = lane / 32,
// e = 0..3) -- the row order of a 32x32 accumulator's 16-row chunk, so it
// pairs with acc_chunk().  r0 % 16 == 0, c0 % 32 == 0.
template <int D, typename E>
__device__ __forceinline__ typename E::v8 lds_tr8(const uint16_t* tile, int r0, int c0, int lane) {
  const int grp = lane >> 4, li = lane & 15;
  const int e = li >> 2, r = li & 3;
  const int g = grp >> 1, half = grp & 1;
  const int rl = 4 * g + e, cl = 16 * half + 4 * r;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + toff2<D>(r0, rl, c0, cl)));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(tile + toff2<D>(r0, rl + 8, c0, cl)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename E::v8, w);
}

// lds_tr8 split into a per-lane part and a compile-time part: with
// tr_lane_offsets(lane, lo, hi), lds_tr8(tile, r0, c0, lane) reads the same
// elements as lds_tr8_at(tile, lo + x, hi + x, r0 * tstride + c0) for any
// column shift x added to both (a multiple of 32).  One pair of lane
// registers then addresses every read of a loop, the rest being immediates.
template <int D, int SW = 2>
__device__ __forceinline__ void tr_lane_offsets(int lane, int& lo, int& hi) {
  const int grp = lane >> 4, li = lane & 15;
  const int rl = 4 * (grp >> 1) + (li >> 2), cl = 16 * (grp & 1) + 4 * (li & 3);
  lo = toff2<D, SW>(0, rl, 0, cl);
  hi = toff2<D, SW>(0, rl + 8, 0, cl);
}
template <typename E>
__device__ __forceinline__ typename E::v8 lds_tr8_at(const uint16_t* tile, int lo, int hi, int imm) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + imm + lo));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + imm + hi));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 w = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(typename E::v8, w);
}

// A pointer that every lane of the wave holds, marked wave-uniform so that
// it lives in scalar registers.  Only for values that are the same in every
// lane.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Raw buffer descriptor over `bytes` bytes from `base` (stride 0; word 3 is
// the gfx9 family's raw-buffer format field, 32-bit data).  Offsets at or
// past `bytes` read as zero instead of reaching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, (int)bytes, 0x00020000);
}

// Direct global -> LDS load of a ROWS x D bf16 tile (rows r0 .. r0+ROWS-1 of
// the n rows of a slice, addressed through `rm` from the slice base `src`)
// into the tile layout, by NT threads.  gfx950's buffer_load_dwordx4 ... lds
// puts the 16 bytes each lane loads at the wave's LDS base (M0) + 16 * lane,
// with no register staging: lane slot p is LDS chunk position p, so the lane
// fetches the logical chunk that the layout stores there; lanes on padding
// slots are switched off.  Rows >= n are filled from row n - 1 (finite
// values that every kernel masks out); the first row r0 must be below n
// (contiguous rows address from row r0).  The loads count on vmcnt; the
// caller waits for them (__syncthreads() does) before reading.  `src`, r0
// and n must be the same in every lane (they are read from the first active
// lane).
//
// Addressing: a descriptor on a scalar base (contiguous rows: the tile's
// first row), a 32-bit per-lane offset and a scalar LDS destination, so a
// load costs no vector instruction beyond its offset, which this general
// form computes per load (clamped only in a tile with rows past the slice's
// end); dma_tile_lanes holds the offsets in registers instead.  The
// global-address form of the load spent a 64-bit vector add per load, the
// compiler keeping each offset as a 64-bit pair.
template <int ROWS, int D, int NT, bool SR>
__device__ __forceinline__ void dma_tile(uint16_t* lds, const uint16_t* src, const RowMap& rm,
                                         int r0, int n, int tid) {
  constexpr int CPR = D / 8, SPR = tstride<D>() / 8, TOTAL = ROWS * SPR;
  static_assert(TOTAL % 64 == 0, "whole waves per tile");
  constexpr int STEPS = (TOTAL + NT - 1) / NT;
  const char* base = uniform_ptr(SR ? src : src + (int64_t)r0 * D);
  // the descriptor's range: the slice from `base` (32-bit byte offsets)
  const int64_t span = SR ? (int64_t)0xffffffff : (int64_t)(n - r0) * (2 * D);
  const __amdgpu_buffer_rsrc_t rsrc = raw_buffer(base, (uint32_t)min(span, (int64_t)0xffffffff));
  const int last = SR ? n - 1 : n - 1 - r0;
  const int w0 = __builtin_amdgcn_readfirstlane(tid & ~63);  // the wave's first slot
  auto issue = [&](auto clamp) {
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      const int wbase = t * NT + w0;
      if (wbase < TOTAL) {
        const int p = t * NT + tid;  // slot wbase + lane
        const int row = p / SPR, phys = p % SPR;
        if (phys < CPR) {
          const int ch = phys ^ ((row >> 2) & 3);
          int rr = SR ? r0 + row : row;
          if constexpr (decltype(clamp)::value) rr = min(rr, last);
          const uint32_t off = SR ? 2u * rm.row(rr) + (uint32_t)(ch * 16)
                                  : (uint32_t)(rr * (2 * D) + ch * 16);  // bytes
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rsrc, (__attribute__((address_space(3))) void*)(lds + wbase * 8), 16, off, 0, 0, 0);
        }
      }
    }
  };
  if (r0 + ROWS <= n)
    issue(std::false_type{});
  else
    issue(std::true_type{});
}

// dma_tile's per-lane addressing for tiles of contiguous rows, computed once
// per kernel and kept in registers: for each load step of a ROWS x D tile,
// the byte offset of the lane's chunk from the tile's first row, or kDmaPad
// on padding slots (past every tile, so the descriptor's range check drops
// those loads and no exec-mask branch is needed).
constexpr uint32_t kDmaPad = 0x40000000u;
template <int ROWS, int D, int NT>
struct DmaLanes {
  static constexpr int CPR = D / 8, SPR = tstride<D>() / 8, TOTAL = ROWS * SPR;
  static constexpr int STEPS = (TOTAL + NT - 1) / NT;
  uint32_t off[STEPS];
  __device__ __forceinline__ explicit DmaLanes(int tid) {
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      const int p = t * NT + tid, row = p / SPR, phys = p % SPR;
      off[t] = (p < TOTAL && phys < CPR) ? (uint32_t)(row * (2 * D) + (phys ^ ((row >> 2) & 3)) * 16)
                                         : kDmaPad;
      // opaque from here on: the compiler keeps the value in a register
      // instead of recomputing it at each load
      asm volatile("" : "+v"(off[t]));
    }
  }
};

// dma_tile with lane offsets precomputed by DmaLanes<ROWS, D, NT> (`off`
// is its array): a tile whose rows all lie below n (every tile of a slice but
// possibly its last) takes one load per step and no vector instruction; the
// rest go through the general path.
template <int ROWS, int D, int NT, bool SR>
__device__ __forceinline__ void dma_tile_lanes(uint16_t* lds, const uint16_t* src, const RowMap& rm,
                                               int r0, int n, int tid, uint32_t* off) {
  using DL = DmaLanes<ROWS, D, NT>;
  if (SR || r0 + ROWS > n) {
    dma_tile<ROWS, D, NT, SR>(lds, src, rm, r0, n, tid);
    return;
  }
  const __amdgpu_buffer_rsrc_t rsrc =
      raw_buffer(uniform_ptr(src + (int64_t)r0 * D), (uint32_t)(ROWS * 2 * D));
  const int w0 = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
  for (int t = 0; t < DL::STEPS; ++t) {
    const int wbase = t * NT + w0;
    if (DL::TOTAL % NT == 0 || wbase < DL::TOTAL) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(lds + wbase * 8), 16, off[t], 0, 0, 0);
    }
  }
}

// The 32 x 32 P / dS staging tile of the backward: row stride 32 elements,
// 8-byte chunk k of row r stored at chunk position k ^ ((r / 2) % 8).  With
// a plain 64-byte stride the column accesses (32 rows, one chunk) were 8-way
// conflicts (SQ_LDS_BANK_CONFLICT).  Measured with an LDS microbenchmark:
// 8-byte accesses of 32 rows at one chunk per 32 lanes, or of 16 rows x 2
// adjacent chunks (the writes from a 16 x 16 accumulator), run at full rate
// under this f and at half rate under f(r) = 2 ((r / 4) % 4) + (r / 16) % 2;
// the transposed reads (4 consecutive rows x 4 chunks per 16 lanes) run at
// the same rate under both.  Element offset of (row r, chunk k).
__device__ __forceinline__ int ds_tile_off(int r, int k) {
  return r * 32 + 4 * (k ^ ((r >> 1) & 7));
}

// Transposed operand read of the dS staging tile, as lds_tr8: free index =
// column c0 + lane % 32, contraction slots = rows r0 + 4g + e, r0 + 8 + 4g + e.
template <typename E>
__device__ __forceinline__ typename E::v8 lds_tr8_ds(const uint16_t* tile, int r0, int c0, int lane) {
  const int grp = lane >> 4, li = lane & 15;
  const int e = li >> 2, r = li & 3;
  const int g = grp >> 1, half = grp & 1;
  const int row = r0 + 4 * g + e, k = (c0 >> 2) + 4 * half + r;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + ds_tile_off(row, k)));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + ds_tile_off(row + 8, k)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename E::v8, w);
}

// Lane offsets of lds_tr8_ds(tile, 16 c, 0, lane), c = 0, 1: the two reads
// at tile + o[c][0] and tile + o[c][1] (see lds_tr8_ds_at).
__device__ __forceinline__ void ds_tr_lane_offsets(int lane, int (&o)[2][2]) {
  const int grp = lane >> 4, li = lane & 15;
  const int e = li >> 2, r = li & 3;
  const int g = grp >> 1, half = grp & 1;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = 16 * c + 4 * g + e, k = 4 * half + r;
    o[c][0] = ds_tile_off(row, k);
    o[c][1] = ds_tile_off(row + 8, k);
  }
}
template <typename E>
__device__ __forceinline__ typename E::v8 lds_tr8_ds_at(const uint16_t* tile, const int (&o)[2]) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o[0]));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o[1]));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename E::v8, w);
}

// Index of key block kb's first dS block within its (b, h): the sum of
// ds_count over the key blocks before kb, summed by the 64 lanes of a wave
// (lane l takes kb' = l, l + 64, ...); every lane returns the total.
__device__ __forceinline__ int64_t ds_offset(const MaskGeom& mg, int kb, int lane) {
  int64_t n = 0;
  for (int k = lane; k < kb; k += 64) n += mg.ds_count(k);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) n += __shfl_xor(n, m);
  return n;
}

// Register-staged tile load: global -> registers now, registers -> LDS (in
// the tile layout) later.  Unlike the direct-to-LDS load, a barrier between
// the two does not wait for the global loads (a barrier waits for LDS
// traffic only), so a tile can be fetched a whole pipeline step before it is
// written.  Rows >= n read as row n - 1 (finite values the kernels mask).
// Rows are addressed through `rm` from the slice base `src`.
template <int ROWS, int D, int NT>
struct RegTile {
  static constexpr int CPR = D / 8, TOTAL = ROWS * CPR, CH = (TOTAL + NT - 1) / NT;
  uint4 r[CH];

  // a uniform base (contiguous rows: the tile's first row) plus a 32-bit
  // per-lane byte offset, the scalar-base form of the load (one address
  // register per load and no 64-bit address arithmetic per lane)
  template <bool SR>
  __device__ __forceinline__ void load(const uint16_t* src, const RowMap& rm, int r0, int n,
                                       int tid) {
    const char* base = reinterpret_cast<const char*>(SR ? src : src + (int64_t)r0 * D);
    const int last = SR ? n - 1 : n - 1 - r0;
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int c = tid + t * NT;
      if (TOTAL % NT == 0 || c < TOTAL) {
        const int row = min((SR ? r0 : 0) + c / CPR, last);
        const uint32_t off = 2u * ((SR ? rm.row(row) : (uint32_t)row * D) + (uint32_t)(c % CPR) * 8);
        r[t] = *reinterpret_cast<const uint4*>(base + off);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int c = tid + t * NT;
      if (TOTAL % NT == 0 || c < TOTAL)
        *reinterpret_cast<uint4*>(lds + toff<D>(c / CPR, (c % CPR) * 8)) = r[t];
    }
  }
};

// Direct global -> LDS load of 64 fp32 values by one wave: lanes 0..31 take
// a[r0 + lane], lanes 32..63 take b[r0 + lane - 32] (indices clamped to
// n - 1), landing at lds[lane].
__device__ __forceinline__ void dma_rows_f32x2(float* lds, const float* a, const float* b, int r0,
                                               int n, int lane) {
  const int r = min(r0 + (lane & 31), n - 1);
  const float* g = (lane < 32 ? a : b) + r;
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// Global -> register MFMA operand of one row (lane l: row l % 32, chunks
// 2kc + l / 32); rows that are not valid read as zero.
template <int D, typename E>
__device__ __forceinline__ void load_operand_rows(typename E::v8 (&op)[D / 16], const uint16_t* rowp,
                                                  bool valid, int gq) {
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    if (valid) {
      op[kc] = *reinterpret_cast<const typename E::v8*>(rowp + 16 * kc + 8 * gq);
    } else {
      op[kc] = typename E::v8{};
    }
  }
}

// Write a transposed accumulator set (accumulator rows = the d columns, this
// lane's accumulator column = tile row `row`) into an LDS tile as
// E, scaled by `mul`: element (row, 32*db + 8*i + 4*gq + j).  Output rows
// go through LDS so that store_tile() writes them with coalesced 16-byte
// stores (storing one row per lane would scatter 8-byte pieces over 32 rows
// per instruction).
template <int D, typename E>
__device__ __forceinline__ void acc_to_lds(uint16_t* tile, int row, const f32x16 (&acc)[D / 32],
                                           float mul, int gq) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint2*>(tile + toff2<D>(0, row, 32 * db, 8 * i + 4 * gq)) =
          pack4<E>(acc[db][4 * i] * mul, acc[db][4 * i + 1] * mul, acc[db][4 * i + 2] * mul,
                   acc[db][4 * i + 3] * mul);
}

// acc_to_lds for NB of the D / 32 column blocks, starting at column c0 (a
// multiple of 32): element (row, c0 + 32*db + 8*i + 4*gq + j) from acc[db].
template <int D, typename E, int NB>
__device__ __forceinline__ void acc_to_lds_cols(uint16_t* tile, int row, const f32x16 (&acc)[NB],
                                                int c0, float mul, int gq) {
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint2*>(tile + toff2<D>(0, row, c0 + 32 * db, 8 * i + 4 * gq)) =
          pack4<E>(acc[db][4 * i] * mul, acc[db][4 * i + 1] * mul, acc[db][4 * i + 2] * mul,
                   acc[db][4 * i + 3] * mul);
}

// LDS -> global copy of a ROWS x D tile to rows r0 .. of the n rows of a
// slice (slice base `dst`, rows addressed through `rm`) by NT threads, 16
// bytes per lane per step, consecutive lanes on consecutive addresses of a
// row; rows >= n are not written.  The stores are non-temporal: every output
// tile is written once and not read back by the kernel that writes it, and
// streaming it past the caches keeps the dirty lines of one kernel's outputs
// from being written back while the next kernel streams its inputs (measured
// on MI355X: Hiera mask-unit forward 71 -> 52 us when run after the backward,
// fused backward 103 -> 96 us).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int ROWS, int D, int NT, bool SR>
__device__ __forceinline__ void store_tile(uint16_t* dst, const RowMap& rm, int r0, int n,
                                           const uint16_t* lds, int tid) {
  constexpr int CPR = D / 8, TOTAL = ROWS * CPR, CH = (TOTAL + NT - 1) / NT;
#pragma unroll
  for (int t = 0; t < CH; ++t) {
    const int c = tid + t * NT;
    const int row = c / CPR, col = (c % CPR) * 8;
    if (c < TOTAL && r0 + row < n)
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(lds + toff<D>(row, col)),
          reinterpret_cast<u32x4*>(dst + (SR ? (int64_t)rm.row(r0 + row) : (int64_t)(r0 + row) * D) + col));
  }
}

}  // namespace
}  // namespace attn
