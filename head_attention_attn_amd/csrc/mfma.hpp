// mfma.hpp -- CDNA4 (gfx950) building blocks for the 16-bit (bf16 and fp16)
// attention kernels.  The kernels are templates over an element type E, Bf16
// or F16 below: storage is 16 bits either way, E supplies the MFMA operand
// vector, the MFMA and the fp32 -> 16-bit conversion (round to nearest even).
//
// v_mfma_f32_32x32x16_bf16 / _f16 lane layout (checked on gfx950 hardware):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) + s, s = 0..7
//   B (16 x 32): lane l holds col l%32, k = 8*(l/32) + s
//   C (32 x 32): lane l holds col l%32, rows 8*i + 4*(l/32) + j in acc[4*i + j]
// v_mfma_f32_16x16x32_bf16 / _f16 (checked on gfx950 hardware):
//   A (16 x 32): lane l holds row l%16, k = 8*(l/16) + s
//   B (32 x 16): lane l holds col l%16, k = 8*(l/16) + s
//   C (16 x 16): lane l holds col l%16, rows 4*(l/16) + j in acc[j]
// The contraction index k may be permuted freely as long as A and B agree;
// the kernels use that to feed an accumulator straight back in as an operand.
//
// ds_read_b64_tr_b16 (LDS transpose read, 16-bit elements): within each group
// of 16 lanes, with source lane 4*e + r pointing at 4 consecutive elements
// M[4e + r][0..3], destination lane i receives M[4e + i/4][i%4] for e = 0..3.
// Pointing source lane 4e + r at row (r0 + e), column (c0 + 4r) of a row-major
// tile therefore gives lane i the four elements (r0 + e, c0 + i), e = 0..3: a
// column read of a row-major tile, which is what an MFMA operand whose
// contraction runs along the tile's rows needs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// element types of the 16-bit kernels
struct Bf16 {
  typedef __bf16 scalar;
  typedef bf16x8 v8;
  typedef bf16x4 v4;
  static __device__ __forceinline__ f32x16 mfma(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(const v8& a, const v8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

struct F16 {
  typedef _Float16 scalar;
  typedef f16x8 v8;
  typedef f16x4 v4;
  static __device__ __forceinline__ f32x16 mfma(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(const v8& a, const v8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <typename E>
__device__ __forceinline__ f32x16 mfma32(const typename E::v8& a, const typename E::v8& b,
                                         const f32x16& c) {
  return E::mfma(a, b, c);
}
template <typename E>
__device__ __forceinline__ f32x4 mfma16(const typename E::v8& a, const typename E::v8& b,
                                        const f32x4& c) {
  return E::mfma16(a, b, c);
}

// Accumulator entries 8c .. 8c+7 of a 32x32 tile, rounded to E: the rows
// (8*(2c) + 4g + j, 8*(2c+1) + 4g + j) of chunk c in the order the transposed LDS read
// uses, ready to be the other operand of a contraction over those rows.
template <typename E>
__device__ __forceinline__ typename E::v8 acc_chunk(const f32x16& acc, int c) {
  f32x8 v;
  #pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = acc[8 * c + s];
  return __builtin_convertvector(v, typename E::v8);
}

template <typename E>
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  typename E::v4 h = __builtin_convertvector(v, typename E::v4);
  return __builtin_bit_cast(uint2, h);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x on lane l combined with x on lane l ^ 32 (the same row's other half in
// the MFMA accumulator layout).  v_permlane32_swap of x with itself leaves
// the lower-half value in one result and the upper-half value in the other
// on every lane, with no LDS round trip.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Masked and unmasked instances of a per-tile loop: f(std::true_type{}) when
// `masked`, else f(std::false_type{}).  The tile-level test is one uniform
// branch; the masked instance tests every element without branches (bitwise
// tests and selects) and the unmasked one has no per-element test at all.
template <typename F>
__device__ __forceinline__ auto with_mask(bool masked, F&& f) {
  if (masked) return f(std::true_type{});
  return f(std::false_type{});
}

// Wave index within the workgroup, marked wave-uniform: everything derived
// from it (the wave's rows or keys, tile visibility, skip decisions) then
// lives in scalar registers and branches on it are uniform, instead of being
// treated as per-lane values with exec-mask control flow.
__device__ __forceinline__ int wave_id(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }

}  // namespace attn
