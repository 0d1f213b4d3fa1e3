// premix.hip -- IHA pseudo-token construction ("IHA-CUDA: Interleaved Head
// Attention Kernels for Hopper GPUs", section "Pseudo-Token Mixing"):
//
//   Out[h, p] = sum_s W[h, p, s] * X[s]      at every (batch, position, feature)
//   dX        = W^T dOut                      (the transposed map)
//   dW[h,p,s] = sum over (b, n, feature) of dOut[h, p] * X[s]
//
// Layouts: X, dX [B][N][H][d]; W [H][P][H] (the input type); Out, dOut
// [B][H][N][P][d] (per head the N * P pseudo-tokens t = n * P + p); dW
// [H][P][H] fp32.
//
// The map is memory-bound (a 16-bit input row of H*d elements becomes H*P*d
// output elements), but at every position it is a small dense contraction
// over heads -- (H*P) x H by H x d -- which runs on the MFMA units at a
// negligible fraction of their rate (fp32 FMAs on the vector ALUs would take
// about as long as the memory traffic).  One workgroup has one wave per 32
// features; it walks positions b * N + n = blockIdx.x, blockIdx.x + grid, ...
// For each position the X rows (H of them, padded to 32 with finite copies
// that the zero-padded W operand cancels) go to LDS, every wave computes its
// 32 features of all H*P outputs with v_mfma_f32_32x32x16 (accumulator
// C[feature][(h,p)], contraction over s read with the LDS transpose read),
// the results go through LDS and leave as whole 2 d-byte rows.
//
// Backward: per position, dOut (H*P rows) and X (H rows) in LDS; dW partial
// sums C[(h,p)][s] (contraction over the wave's 32 features) stay in
// registers for all the workgroup's positions; dX = C[feature][s] with the
// contraction over (h,p) read transposed from the dOut tile.  At the end the
// waves add their partial dW into one fp32 LDS block in wave order and the
// workgroup writes it to the workspace; a second kernel sums the partials in
// workgroup order.  No atomics: results are bitwise deterministic.  (The
// pages' backward reduces dW with atomics.)
#include "attn_common.hpp"
#include "bf16_tile.hpp"

namespace attn {

namespace {

// at most 32 source heads (one 32-wide MFMA column, two k-steps of 16) and
// H * P <= 128 output heads (four 32-row tiles); the host checks both
constexpr int kMaxHP = 128;

// W operand of the forward for output tile nt, k-step ks: an MFMA B operand
// (column (h,p) = 32 nt + lane % 32) whose contraction slots follow the row
// order of lds_tr8 -- slot e < 4 is s = 16 ks + 4 g + e, slot e >= 4 is
// s = 16 ks + 8 + 4 g + e - 4 (g = lane / 32).  Zero outside H and H * P.
template <typename E>
__device__ __forceinline__ typename E::v8 w_operand_fwd(const uint16_t* w, int H, int HP, int nt,
                                                        int ks, int lane) {
  typename E::v8 op = {};
  const int m = 32 * nt + (lane & 31), g = lane >> 5;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int s = 16 * ks + (e < 4 ? 4 * g + e : 8 + 4 * g + e - 4);
    if (m < HP && s < H) {
      const uint16_t bits = w[m * H + s];
      op[e] = __builtin_bit_cast(typename E::scalar, bits);
    }
  }
  return op;
}

// W^T operand of dX for k-step ks: column s = lane % 32, contraction slots
// over (h,p) in lds_tr8 row order.  Zero outside.
template <typename E>
__device__ __forceinline__ typename E::v8 w_operand_bwd(const uint16_t* w, int H, int HP, int ks,
                                                        int lane) {
  typename E::v8 op = {};
  const int s = lane & 31, g = lane >> 5;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int m = 16 * ks + (e < 4 ? 4 * g + e : 8 + 4 * g + e - 4);
    if (m < HP && s < H) {
      const uint16_t bits = w[m * H + s];
      op[e] = __builtin_bit_cast(typename E::scalar, bits);
    }
  }
  return op;
}

// Row map of the (h,p) rows of one position's output: row r = h * P + p at
// h * (N * P * d) + p * d from the position's first element.
__device__ __forceinline__ RowMap hp_rows(int N, int lp, int D) {
  RowMap rm;
  rm.batch = 0;
  rm.head = 0;
  rm.win = (N << lp) * D;
  rm.tok = D;
  rm.wshift = lp;
  rm.wmask = (1 << lp) - 1;
  return rm;
}

template <typename E, int D>
__global__ __launch_bounds__(2 * D) __attribute__((amdgpu_waves_per_eu(4))) void premix_fwd_kernel(PremixArgs a) {
  constexpr int NT = 2 * D, XE = tile_elems<32, D>();
  // X rows of two positions: the next one streams in (direct-to-LDS) while
  // the current one is computed; named buffers, two positions per loop trip.
  // Outputs are staged 32 rows (h,p) at a time in two alternating buffers,
  // so a tile is computed while the previous one is being stored: 4 tiles
  // of LDS in all, four workgroups per CU.
  __shared__ __attribute__((aligned(16))) uint16_t sX0[XE];
  __shared__ __attribute__((aligned(16))) uint16_t sX1[XE];
  __shared__ __attribute__((aligned(16))) uint16_t sS0[XE];
  __shared__ __attribute__((aligned(16))) uint16_t sS1[XE];
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);  // this wave's 32 features: 32 * wave ..
  const int H = a.H, HP = a.H << a.lp, ntile = (HP + 31) / 32;
  const uint16_t* w = (const uint16_t*)a.w;

  typename E::v8 wop[kMaxHP / 32][2];
#pragma unroll
  for (int nt = 0; nt < kMaxHP / 32; ++nt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) wop[nt][ks] = w_operand_fwd<E>(w, H, HP, nt, ks, lane);

  const RowMap plain{};  // contiguous rows (unused by the SR = false helpers)
  const RowMap rout = hp_rows(a.N, a.lp, D);
  const int64_t npos = (int64_t)a.B * a.N, G = gridDim.x;
  auto fetch = [&](int64_t pos, uint16_t* x_l) {
    dma_tile<32, D, NT, false>(x_l, (const uint16_t*)a.x + pos * H * D, plain, 0, H, tid);
  };
  // one position from x_l: outputs through sS0 / sS1 to global.  Tile nt
  // is written into the buffer tile nt - 2 was stored from; every thread is
  // past that store since it passed the barrier of tile nt - 1 (the first
  // tile of a position follows the position's own barrier).
  auto position = [&](int64_t pos, const uint16_t* x_l) {
    const int b = (int)(pos / a.N), n = (int)(pos % a.N);
    uint16_t* out = (uint16_t*)a.out + ((int64_t)b * H * a.N + n) * ((int64_t)D << a.lp);
#pragma unroll
    for (int nt = 0; nt < kMaxHP / 32; ++nt) {
      if (nt >= ntile) break;
      uint16_t* st = (nt & 1) ? sS1 : sS0;
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        if (16 * ks < H)
          acc = mfma32<E>(lds_tr8<D, E>(x_l, 16 * ks, 32 * wave, lane), wop[nt][ks], acc);
      // C[feature 32 wave + 8 i + 4 gq + j][(h,p) 32 nt + lane % 32]
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint2*>(st + toff2<D>(0, lane & 31, 32 * wave, 8 * i + 4 * gq)) =
            pack4<E>(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
      __syncthreads();  // staging complete (and, at nt = 0, the prefetch landed)
      store_tile<32, D, NT, true>(out, rout, 32 * nt, HP, st, tid);
    }
  };

  int64_t pos = blockIdx.x;
  fetch(pos, sX0);
  for (;;) {
    __syncthreads();  // X of pos in sX0; sX1 and sS free
    if (pos + G < npos) fetch(pos + G, sX1);
    position(pos, sX0);
    pos += G;
    if (pos >= npos) break;
    __syncthreads();  // X of pos in sX1; sX0 and sS free
    if (pos + G < npos) fetch(pos + G, sX0);
    position(pos, sX1);
    pos += G;
    if (pos >= npos) break;
  }
}

template <typename E, int D>
__global__ __launch_bounds__(2 * D) void premix_bwd_kernel(PremixArgs a) {
  constexpr int NT = 2 * D, NW = D / 32, XE = tile_elems<32, D>(), YE = tile_elems<kMaxHP, D>();
  __shared__ __attribute__((aligned(16))) uint16_t sX[XE];  // X rows, then dX staging
  __shared__ __attribute__((aligned(16))) uint16_t sY[YE];  // dOut rows (h,p)
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);
  const int H = a.H, HP = a.H << a.lp, ntile = (HP + 31) / 32, nks = (HP + 15) / 16;
  const uint16_t* w = (const uint16_t*)a.w;

  typename E::v8 wtop[kMaxHP / 16];
#pragma unroll
  for (int ks = 0; ks < kMaxHP / 16; ++ks) wtop[ks] = w_operand_bwd<E>(w, H, HP, ks, lane);
  f32x16 dw[kMaxHP / 32];
#pragma unroll
  for (int mt = 0; mt < kMaxHP / 32; ++mt) dw[mt] = f32x16{};

  const RowMap plain{};
  const RowMap rout = hp_rows(a.N, a.lp, D);
  const int64_t npos = (int64_t)a.B * a.N;
  for (int64_t pos = blockIdx.x; pos < npos; pos += gridDim.x) {
    const int b = (int)(pos / a.N), n = (int)(pos % a.N);
    const uint16_t* dout =
        (const uint16_t*)a.dout + ((int64_t)b * H * a.N + n) * ((int64_t)D << a.lp);
    dma_tile<kMaxHP, D, NT, true>(sY, dout, rout, 0, HP, tid);
    dma_tile<32, D, NT, false>(sX, (const uint16_t*)a.x + pos * H * D, plain, 0, H, tid);
    __syncthreads();
    // dW[(h,p)][s] += sum over this wave's 32 features of dOut[(h,p)][c] X[s][c]
#pragma unroll
    for (int mt = 0; mt < kMaxHP / 32; ++mt) {
      if (mt >= ntile) break;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        dw[mt] = mfma32<E>(lds_row8<D, E>(sY, 32 * mt, lane & 31, 2 * wave + kc, gq),
                           lds_row8<D, E>(sX, 0, lane & 31, 2 * wave + kc, gq), dw[mt]);
    }
    // dX[c][s] = sum over (h,p) of dOut^T[c][(h,p)] W[(h,p)][s]
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < kMaxHP / 16; ++ks) {
      if (ks >= nks) break;
      acc = mfma32<E>(lds_tr8<D, E>(sY, 16 * ks, 32 * wave, lane), wtop[ks], acc);
    }
    __syncthreads();  // every wave is past its reads of sX
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint2*>(sX + toff2<D>(0, lane & 31, 32 * wave, 8 * i + 4 * gq)) =
          pack4<E>(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    __syncthreads();
    store_tile<32, D, NT, false>((uint16_t*)a.dx + pos * H * D, plain, 0, H, sX, tid);
    __syncthreads();
  }

  // the waves' partial dW, added in wave order into one fp32 block in LDS
  // (sY is free), then this workgroup's partial to the workspace
  float* sW = reinterpret_cast<float*>(sY);  // [kMaxHP][32]
  static_assert(YE * 2 >= kMaxHP * 32 * 4, "dW block fits in the dOut tile");
  for (int wv = 0; wv < NW; ++wv) {
    if (wave == wv) {
#pragma unroll
      for (int mt = 0; mt < kMaxHP / 32; ++mt) {
        if (mt >= ntile) break;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = 32 * mt + 8 * (e >> 2) + 4 * gq + (e & 3);
          float* p = sW + m * 32 + (lane & 31);
          *p = wv == 0 ? dw[mt][e] : *p + dw[mt][e];
        }
      }
    }
    __syncthreads();
  }
  float* part = a.dw_part + (int64_t)blockIdx.x * HP * H;
  for (int e = tid; e < HP * H; e += NT) part[e] = sW[(e / H) * 32 + e % H];
}

// dW[e] = sum over workgroups g (in order) of part[g][e]: 64 elements per
// workgroup, the 16 waves taking g = wave, wave + 16, ...; their 16 sums are
// then added in wave order.
__global__ __launch_bounds__(1024) void premix_dw_reduce_kernel(const float* __restrict__ part,
                                                                float* __restrict__ dw, int nelem,
                                                                int nparts) {
  __shared__ float sP[16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  float acc = 0.f;
  // (unrolled so that the loads of several partials are in flight at once;
  // the additions keep their order)
  if (e < nelem) {
#pragma unroll 16
    for (int g = wave; g < nparts; g += 16) acc += part[(int64_t)g * nelem + e];
  }
  sP[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && e < nelem) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += sP[k][lane];
    dw[e] = t;
  }
}

template <typename E, int D>
int fwd_d(const PremixArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((premix_fwd_kernel<E, D>), dim3(a.grid), dim3(2 * D), 0, s, a);
  return (int)hipGetLastError();
}

template <typename E, int D>
int bwd_d(const PremixArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((premix_bwd_kernel<E, D>), dim3(a.grid), dim3(2 * D), 0, s, a);
  int err = (int)hipGetLastError();
  if (err) return err;
  const int nelem = (a.H << a.lp) * a.H;
  hipLaunchKernelGGL(premix_dw_reduce_kernel, dim3((nelem + 63) / 64), dim3(1024), 0, s,
                     a.dw_part, a.dw, nelem, a.grid);
  return (int)hipGetLastError();
}

template <typename E>
int fwd_e(const PremixArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return fwd_d<E, 64>(a, s);
    case 96: return fwd_d<E, 96>(a, s);
    case 128: return fwd_d<E, 128>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

template <typename E>
int bwd_e(const PremixArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return bwd_d<E, 64>(a, s);
    case 96: return bwd_d<E, 96>(a, s);
    case 128: return bwd_d<E, 128>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_premix_fwd(const PremixArgs& a, bool f16, int d, hipStream_t s) {
  return f16 ? fwd_e<F16>(a, d, s) : fwd_e<Bf16>(a, d, s);
}

int launch_premix_bwd(const PremixArgs& a, bool f16, int d, hipStream_t s) {
  return f16 ? bwd_e<F16>(a, d, s) : bwd_e<Bf16>(a, d, s);
}

}  // namespace attn
