// attn_bf16_short.hip -- fused one-pass backward for short key sequences:
// every key of a (b, h) fits one workgroup (Nk <= 224, d = 64 or 96), as in
// the global-attention stages of Hiera-Base at 224x224 ("hiera-optim 0.1.0",
// Results, and the sdist's mask_unit.py on the global-attention stages; the
// 14x14 grid has 196 tokens).  Any mask.
//
// The backward of FlashAttention-2 ("IHA-CUDA", Repository Structure:
// preprocess, flash backward, postprocess) needs three passes over HBM when
// the keys of a row span several workgroups: the row sums D_i, then dK/dV,
// then dQ.  With all keys of a (b, h) in one workgroup they collapse into one
// pass that reads Q, K, V, dO and lse once and writes dQ, dK, dV once: O is
// not read and no workspace is used.
//
// Workgroup = one (b, h), 8 waves, K and V of the (b, h) in LDS.  Waves 0..6
// own 32 keys each (dK^T and dV^T accumulate in registers over the whole
// call); wave 7 owns dQ.  The query rows go by in slabs of 32:
//   key waves:  S = Q K^T, dP = dO V^T, P = exp(S scale - lse) for the slab;
//               partial row sums sum_j P_ij dP_ij over their 32 keys, reduced
//               across the half-wave and left in LDS;
//   barrier;    D_i = sum of the 7 partials (equal to sum_c dO_ic O_ic, the
//               "dPsum" of the pre-pass), dS = P (dP - D), written to LDS as
//               [key][query] tiles; dV^T += dO^T P, dK^T += Q^T dS;
//   barrier;    the dQ wave: dQ^T = K^T dS^T over all keys (K in LDS), rows
//               staged through LDS and stored -- while the key waves start
//               the next slab.
// Q / dO slabs are fetched two slabs ahead into registers (a barrier does not
// wait for register loads) and written to one of two LDS buffers one slab
// ahead.  No atomics: results are bitwise deterministic.
#include "attn_common.hpp"
#include "bf16_tile.hpp"

namespace attn {

namespace {

constexpr int kKeyWaves = kShortKeys / 32;  // 7
constexpr int kNT = 64 * (kKeyWaves + 1);   // 512 threads

// v_swizzle within each 32-lane half: lane l reads lane l ^ m (bitmask mode,
// and-mask 31, or-mask 0, xor-mask m)
template <int M>
__device__ __forceinline__ float swz_xor(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (M << 10) | 0x1f));
}

// One halving step of a half-wave reduction: of the 2N values a lane holds,
// it keeps the half picked by lane bit M and adds the partner's (lane ^ M)
// copy of that half.
template <int M, int N>
__device__ __forceinline__ void halve(float (&v)[16], bool hi) {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float send = hi ? v[k] : v[k + N];
    const float keep = hi ? v[k + N] : v[k];
    v[k] = keep + swz_xor<M>(send);
  }
}

// Row sums of a 32 x 32 accumulator (rows 8(e/4) + 4g + e%4 for entry e,
// g = lane / 32, column = lane % 32) over its 32 columns: 16 exchanges
// instead of 5 per entry.  Lane l returns the sum of entry e = (l % 32) / 2
// of its half, i.e. of row 8(e/4) + 4g + e%4.
__device__ __forceinline__ float row_sums_halves(const f32x16& acc, int lane) {
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = acc[e];
  halve<16, 8>(v, lane & 16);
  halve<8, 4>(v, lane & 8);
  halve<4, 2>(v, lane & 4);
  halve<2, 1>(v, lane & 2);
  return v[0] + swz_xor<1>(v[0]);
}

template <typename E, int D, bool SR>
__global__ __launch_bounds__(kNT) void bwd_short_kernel(BwdArgs a) {
  using V8 = typename E::v8;
  constexpr int KC = D / 16, DB = D / 32, SE = tile_elems<32, D>();
  __shared__ __attribute__((aligned(16))) uint16_t sK[tile_elems<kShortKeys, D>()];
  __shared__ __attribute__((aligned(16))) uint16_t sV[tile_elems<kShortKeys, D>()];
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[SE];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[SE];
  __shared__ __attribute__((aligned(16))) uint16_t sG0[SE];
  __shared__ __attribute__((aligned(16))) uint16_t sG1[SE];
  __shared__ __attribute__((aligned(16))) uint16_t sO[SE];                  // dQ rows, staged
  __shared__ __attribute__((aligned(16))) uint16_t sDS[kKeyWaves * 1024];  // dS^T per key block
  __shared__ __attribute__((aligned(16))) float sDp[kKeyWaves * 32];       // partial row sums
  __shared__ __attribute__((aligned(16))) float sL0[32];                   // lse * log2(e)
  __shared__ __attribute__((aligned(16))) float sL1[32];

  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);
  const int bh = blockIdx.x;
  const int nq = a.nq, nk = a.nk;
  const int nkb = short_key_blocks(nk);  // key blocks, <= kKeyWaves
  const MaskGeom mg = a.mg;
  const bool dq_wave = wave == kKeyWaves;

  const uint16_t* Q = (const uint16_t*)a.q + rslice<SR, D>(a.rq, bh, a.H, nq);
  const uint16_t* K = (const uint16_t*)a.k + rslice<SR, D>(a.rk, bh, a.H, nk);
  const uint16_t* V = (const uint16_t*)a.v + rslice<SR, D>(a.rv, bh, a.H, nk);
  const uint16_t* dO = (const uint16_t*)a.dout + rslice<SR, D>(a.rdo, bh, a.H, nq);
  const float* LSE = a.lse + (int64_t)bh * nq;

  // every key block's K and V rows (32-row tiles laid end to end are one tall
  // tile: the layout's swizzle repeats every 16 rows).  The dQ products run
  // over all kKeyWaves blocks, unrolled: blocks past the keys hold a copy of
  // the last key block (short_k_block_row; a tile load must start at a row
  // < nk) and their dS stays zero, as do their partial row sums.
#pragma unroll
  for (int b = 0; b < kKeyWaves; ++b)
    dma_tile<32, D, kNT, SR>(sK + b * SE, K, a.rk, short_k_block_row(b, nk), nk, tid);
  for (int b = 0; b < nkb; ++b) dma_tile<32, D, kNT, SR>(sV + b * SE, V, a.rv, 32 * b, nk, tid);
  for (int i = tid; i < kKeyWaves * 1024 / 8; i += kNT) reinterpret_cast<uint4*>(sDS)[i] = uint4{0, 0, 0, 0};
  for (int i = tid; i < kKeyWaves * 32; i += kNT) sDp[i] = 0.f;

  // key waves: this lane's key and the query rows that see it
  const int myk = 32 * wave + (lane & 31);
  const bool kvalid = !dq_wave && myk < nk;
  const int clo = kvalid ? mg.col_lo(myk) : nq, chi = kvalid ? mg.col_hi(myk) : nq;
  const bool wave_keys = !dq_wave && 32 * wave < nk;

  // Q / dO slabs through registers: slab s + 2 is fetched while slab s is
  // worked on, slab s + 1 is written to LDS
  RegTile<32, D, kNT> pq, pg;
  float plse = 0.f;
  auto fetch = [&](int s) {
    pq.template load<SR>(Q, a.rq, 32 * s, nq, tid);
    pg.template load<SR>(dO, a.rdo, 32 * s, nq, tid);
    if (tid < 32) plse = LSE[min(32 * s + tid, nq - 1)];
  };
  auto commit = [&](uint16_t* q_l, uint16_t* g_l, float* l_l, int s) {
    pq.store(q_l, tid);
    pg.store(g_l, tid);
    if (tid < 32) l_l[tid] = 32 * s + tid < nq ? plse * kLog2e : 0.f;
  };
  const int nslab = (nq + 31) / 32;
  fetch(0);
  commit(sQ0, sG0, sL0, 0);
  if (nslab > 1) fetch(1);

  f32x16 acc0[DB], acc1[DB];  // key waves: dK^T, dV^T; the dQ wave: dQ^T of a slab in acc0
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    acc0[db] = f32x16{};
    acc1[db] = f32x16{};
  }
  const float sl2 = a.scale * kLog2e;
  uint16_t* dQ = (uint16_t*)a.dq + rslice<SR, D>(a.rdq, bh, a.H, nq);
  __syncthreads();

  for (int s = 0; s < nslab; ++s) {
    const bool odd = s & 1;
    const uint16_t* q_l = odd ? sQ1 : sQ0;
    const uint16_t* g_l = odd ? sG1 : sG0;
    const float* l_l = odd ? sL1 : sL0;
    const int i0 = 32 * s;
    f32x16 p = f32x16{}, dp = f32x16{};
    if (wave_keys) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        p = mfma32<E>(lds_row8<D, E>(q_l, 0, lane & 31, kc, gq), lds_row8<D, E>(sK, 32 * wave, lane & 31, kc, gq), p);
        dp = mfma32<E>(lds_row8<D, E>(g_l, 0, lane & 31, kc, gq), lds_row8<D, E>(sV, 32 * wave, lane & 31, kc, gq), dp);
      }
      const int bk0 = 32 * wave;
      const bool full = bk0 + 32 <= nk && mg.tile_full(i0, i0 + 32, bk0, bk0 + 32);
      f32x16 t;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 L4 = *reinterpret_cast<const f32x4*>(&l_l[8 * i + 4 * gq]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * i + j;
          const int qi = i0 + 8 * i + 4 * gq + j;
          const bool vis = full || (qi >= clo && qi < chi);
          const float pe = vis ? fast_exp2(fmaf(p[e], sl2, -L4[j])) : 0.f;
          p[e] = pe;
          t[e] = pe * dp[e];
        }
      }
      const float rs = row_sums_halves(t, lane);
      const int e = (lane & 31) >> 1;
      if (!(lane & 1)) sDp[32 * wave + 8 * (e >> 2) + 4 * gq + (e & 3)] = rs;
    }
    if (s + 1 < nslab) {
      if (odd) commit(sQ0, sG0, sL0, s + 1);
      else commit(sQ1, sG1, sL1, s + 1);
    }
    if (s + 2 < nslab) fetch(s + 2);
    __syncthreads();  // partial row sums and the next slab in LDS

    if (wave_keys) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 D4 = *reinterpret_cast<const f32x4*>(&sDp[8 * i + 4 * gq]);
#pragma unroll
        for (int b = 1; b < kKeyWaves; ++b) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sDp[32 * b + 8 * i + 4 * gq]);
          D4 += x;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[4 * i + j] = p[4 * i + j] * (dp[4 * i + j] - D4[j]);
        // dS^T tile of this key block: row = key, 8-byte chunk 2i + g =
        // queries 8i + 4g .. +3
        *reinterpret_cast<uint2*>(sDS + 1024 * wave + ds_tile_off(lane & 31, 2 * i + gq)) =
            pack4<E>(dp[4 * i], dp[4 * i + 1], dp[4 * i + 2], dp[4 * i + 3]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const V8 pop = acc_chunk<E>(p, c);
        const V8 dsop = acc_chunk<E>(dp, c);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          acc1[db] = mfma32<E>(lds_tr8<D, E>(g_l, 16 * c, 32 * db, lane), pop, acc1[db]);
          acc0[db] = mfma32<E>(lds_tr8<D, E>(q_l, 16 * c, 32 * db, lane), dsop, acc0[db]);
        }
      }
    }
    __syncthreads();  // dS of the slab in LDS

    if (dq_wave) {
      f32x16 (&dqa)[DB] = acc0;
#pragma unroll
      for (int db = 0; db < DB; ++db) dqa[db] = f32x16{};
#pragma unroll
      for (int b = 0; b < kKeyWaves; ++b) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const V8 dsop = lds_tr8_ds<E>(sDS + 1024 * b, 16 * h, 0, lane);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            dqa[db] = mfma32<E>(lds_tr8<D, E>(sK, 32 * b + 16 * h, 32 * db, lane), dsop, dqa[db]);
        }
      }
      // rows through LDS for whole-row stores; this wave alone writes and
      // reads sO, and a wave's LDS accesses complete in order
      acc_to_lds<D, E>(sO, lane & 31, dqa, a.scale, gq);
      __builtin_amdgcn_wave_barrier();
      store_tile<32, D, 64, SR>(dQ, a.rdq, i0, nq, sO, lane);
    }
  }

  // dK, then dV: rows through the K tile (no wave reads K after the loop)
  __syncthreads();
  uint16_t* dK = (uint16_t*)a.dk + rslice<SR, D>(a.rdk, bh, a.H, nk);
  uint16_t* dV = (uint16_t*)a.dv + rslice<SR, D>(a.rdv, bh, a.H, nk);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (pass) __syncthreads();
    if (wave_keys) acc_to_lds<D, E>(sK, 32 * wave + (lane & 31), pass ? acc1 : acc0, pass ? 1.f : a.scale, gq);
    __syncthreads();
    store_tile<kShortKeys, D, kNT, SR>(pass ? dV : dK, pass ? a.rdv : a.rdk, 0, nk, sK, tid);
  }
}

template <typename E, int D>
int bwd_d(const BwdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.B * a.H));
  if (rows_plain(a, D))
    hipLaunchKernelGGL((bwd_short_kernel<E, D, false>), grid, dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_short_kernel<E, D, true>), grid, dim3(kNT), 0, s, a);
  return (int)hipGetLastError();
}

template <typename E>
int bwd_e(const BwdArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return bwd_d<E, 64>(a, s);
    case 96: return bwd_d<E, 96>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_bwd_16_short(const BwdArgs& a, bool f16, int d, hipStream_t s) {
  return f16 ? bwd_e<F16>(a, d, s) : bwd_e<Bf16>(a, d, s);
}

}  // namespace attn
