// bf16_tile.hpp -- tile staging and operand helpers shared by the bf16
// attention kernels (global -> register -> LDS tile copies, MFMA operand
// loads of whole rows, bf16 row stores of transposed accumulators).
#pragma once

#include "attn_common.hpp"
#include "mfma.hpp"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// Cooperative global -> register -> LDS staging of a ROWS x D bf16 tile whose
// rows start at r0 of a [n][D] matrix; rows >= n read as zero.
template <int ROWS, int D, int NT>
struct TileLoader {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int TOTAL = ROWS * CPR;
  static constexpr int CH = (TOTAL + NT - 1) / NT;    // chunks per thread
  uint4 r[CH];

  __device__ __forceinline__ void load(const uint16_t* src, int r0, int n, int tid) {
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int c = tid + t * NT;
      const int row = c / CPR, col = (c % CPR) * 8;
      const int gr = r0 + row;
      r[t] = (c < TOTAL && gr < n)
                 ? *reinterpret_cast<const uint4*>(src + (int64_t)gr * D + col)
                 : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int stride, int tid) const {
#pragma unroll
    for (int t = 0; t < CH; ++t) {
      const int c = tid + t * NT;
      const int row = c / CPR, col = (c % CPR) * 8;
      if (c < TOTAL) *reinterpret_cast<uint4*>(lds + row * stride + col) = r[t];
    }
  }
};

// Direct global -> LDS copy of a ROWS x D bf16 tile whose rows start at r0 of
// a [n][D] matrix, into the padded LDS layout of row stride D + 8 (gfx950
// global_load_lds_dwordx4: the 16 bytes each lane loads land at the wave's
// LDS base + 16 * lane, with no register staging).  The tile is ROWS * SPR
// 16-byte slots, SPR = D / 8 + 1 per row; slot p is row p / SPR, column chunk
// p % SPR.  The padding slot of each row receives that row's first chunk and
// rows >= n receive row n - 1: finite values that every kernel masks out.
// The LDS array must hold lds_slots(ROWS, D) slots.  Completion is waited for
// by the caller (s_waitcnt vmcnt(0), which __syncthreads() implies).
__host__ __device__ constexpr int lds_slots(int rows, int d) {
  return ((rows * (d / 8 + 1) + 63) / 64) * 64;
}

template <int ROWS, int D, int NT>
__device__ __forceinline__ void dma_tile(uint16_t* lds, const uint16_t* src, int r0, int n,
                                         int tid) {
  constexpr int SPR = D / 8 + 1, TOTAL = ROWS * SPR;
  constexpr int STEPS = (TOTAL + NT - 1) / NT;
#pragma unroll
  for (int t = 0; t < STEPS; ++t) {
    const int wbase = t * NT + (tid & ~63);  // first slot of this wave's 64
    if (wbase < TOTAL) {
      const int p = t * NT + tid;
      const int row = p / SPR, ch = p % SPR;
      const int gr = min(r0 + row, n - 1);
      const uint16_t* g = src + (int64_t)gr * D + (ch == SPR - 1 ? 0 : ch * 8);
      if (p < TOTAL)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)g,
            (__attribute__((address_space(3))) void*)(lds + wbase * 8), 16, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_operand_rows(bf16x8 (&op)[D / 16], const uint16_t* rowp,
                                                  bool valid, int gq) {
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    if (valid) {
      op[kc] = *reinterpret_cast<const bf16x8*>(rowp + 16 * kc + 8 * gq);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) op[kc][s] = (__bf16)0.0f;
    }
  }
}

// Store a transposed 32-column accumulator block set (columns = this lane's
// row of the output, rows = d) as bf16: d = 32*db + 8*i + 4*gq + j.
template <int D>
__device__ __forceinline__ void store_row_bf16(uint16_t* rowp, const f32x16 (&acc)[D / 32],
                                               float mul, int gq) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint2*>(rowp + 32 * db + 8 * i + 4 * gq) =
          pack_bf16x4(acc[db][4 * i] * mul, acc[db][4 * i + 1] * mul,
                      acc[db][4 * i + 2] * mul, acc[db][4 * i + 3] * mul);
}

// Write a transposed accumulator set (rows = d, this lane's column = output
// row `row` of an LDS tile) into the LDS tile as bf16, scaled by `mul`:
// element (row, 32*db + 8*i + 4*gq + j).  Used to turn per-lane output rows
// into a row-major tile that TileStorer writes out with coalesced 16-byte
// stores (a direct store of one row per lane would scatter 8-byte pieces over
// 32 rows per instruction).
template <int D>
__device__ __forceinline__ void acc_to_lds(uint16_t* tile, int stride, int row,
                                           const f32x16 (&acc)[D / 32], float mul, int gq) {
  uint16_t* rp = tile + row * stride;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint2*>(rp + 32 * db + 8 * i + 4 * gq) =
          pack_bf16x4(acc[db][4 * i] * mul, acc[db][4 * i + 1] * mul,
                      acc[db][4 * i + 2] * mul, acc[db][4 * i + 3] * mul);
}

// Cooperative LDS -> global copy of a ROWS x D bf16 tile to rows r0.. of a
// [n][D] matrix, 16 bytes per lane per step, consecutive lanes on
// consecutive addresses; rows >= n are not written.
template <int ROWS, int D, int NT>
__device__ __forceinline__ void store_tile(uint16_t* dst, int r0, int n, const uint16_t* lds,
                                           int stride, int tid) {
  constexpr int CPR = D / 8, TOTAL = ROWS * CPR, CH = (TOTAL + NT - 1) / NT;
#pragma unroll
  for (int t = 0; t < CH; ++t) {
    const int c = tid + t * NT;
    const int row = c / CPR, col = (c % CPR) * 8;
    if (c < TOTAL && r0 + row < n)
      *reinterpret_cast<uint4*>(dst + (int64_t)(r0 + row) * D + col) =
          *reinterpret_cast<const uint4*>(lds + row * stride + col);
  }
}

}  // namespace
}  // namespace attn
