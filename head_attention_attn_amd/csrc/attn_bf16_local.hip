// attn_bf16_local.hip -- bf16 kernels for attention whose every query row sees
// keys of its own 64-key tile only: block-local (mask-unit) attention with a
// key window w that divides 64 ("hiera-optim 0.1.0" sdist, mask_unit.py,
// MaskUnitAttentionFast: tokens split into independent windows, dense softmax
// attention inside each window), each window holding wq query rows with wq
// dividing w -- wq = w, or fewer when the queries are max-pooled inside the
// window (MaskUnitAttentionFast with q_stride = w / wq).  A tile is then 64
// keys, i.e. 64 / w whole windows, and their QT = 64 wq / w query rows.  Such
// attention is HBM-bound: a 64-token window with d = 96 costs ~4 MFLOP of
// MFMA work against ~100 KB of HBM traffic, so these kernels are built
// around moving each byte once.
//
// Forward: one workgroup per tile, one wave per 32 query rows (QR = 32 or 64
// rows of query buffer, QT of them real).  V of the tile goes to LDS, and K
// too when two waves share it (with one wave, QR = 32, K goes straight into
// the wave's operand registers); each wave keeps 32 query rows as the
// register operand, and the scores of a row are complete after one tile, so
// the softmax is a plain one (exact row max, no rescaling).  Computed
// transposed like the general forward kernel: S^T = K Q^T, O^T = V^T P^T
// with bf16 MFMA 32x32x16.
//
// Backward: one workgroup per tile, Q, K, V and dO staged in LDS once.  The
// dK/dV pass and the dQ pass ("IHA-CUDA", Repository Structure: separate
// backward kernels, no atomic accumulation here) run side by side on
// different waves of the same workgroup: waves 0-1 own 32 keys each
// (dV^T += dO^T P, dK^T += Q^T dS), the waves after them own 32 query rows
// each (dQ^T += K^T dS^T).  Because the tile holds every key a query row can
// see, the row sums D_i = sum_j P_ij dP_ij (equal to sum_c dO_ic O_ic, the
// "dPsum" of the backward pre-pass) are taken by the dQ waves from their own
// P and dP and handed to the dK/dV waves through LDS: O is never read and the
// backward makes one pass over HBM.
#include "attn_common.hpp"
#include "bf16_tile.hpp"

// The forward's waves-per-EU attribute is a register budget; LDS limits some
// instances (wide d, 32-row query tiles) below it, which the compiler reports.
#pragma clang diagnostic ignored "-Wpass-failed"

namespace attn {

namespace {

constexpr int kTile = 64;  // keys per tile

// Tile geometry (LocalTile, attn_common.hpp): tile t holds keys
// [64 t, 64 t + 64) and query rows [QT t, QT t + QT).  Query row r and key c
// of a tile (both counted from the tile's start, which is window-aligned on
// both sides) see each other iff row r is real and r >> lq == c >> lw.  A
// real row's window keys all exist (Nk is a multiple of w), so keys past Nk
// are never visible.

// ------------------------------------------------------------------ forward

// QR: query buffer rows (32 when QT <= 32, else 64); one wave per 32 rows
template <typename E, int D, int QR, bool SR>
__global__ __launch_bounds__(2 * QR) __attribute__((amdgpu_waves_per_eu(3))) void fwd_local_kernel(FwdArgs a, int ntile, int lw, int lq) {
  using V8 = typename E::v8;
  constexpr int NT = 2 * QR, TE = tile_elems<kTile, D>(), KC = D / 16, DB = D / 32;
  // with one wave per tile (QR = 32) the K rows go straight into registers:
  // no wave reads them twice, and half the LDS per tile doubles the tiles
  // (and bytes) in flight per CU
  constexpr bool KREG = QR == 32;
  __shared__ __attribute__((aligned(16))) uint16_t sK[KREG ? 8 : TE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[TE];

  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);
  const int bh = blockIdx.x / ntile;
  const int tile = blockIdx.x % ntile;
  const LocalTile lt = local_tile(tile, a.nq, lw, lq);
  const int tk0 = lt.tk0;

  const uint16_t* Q = (const uint16_t*)a.q + rslice<SR, D>(a.rq, bh, a.H, a.nq);
  const uint16_t* K = (const uint16_t*)a.k + rslice<SR, D>(a.rk, bh, a.H, a.nk);
  const uint16_t* V = (const uint16_t*)a.v + rslice<SR, D>(a.rv, bh, a.H, a.nk);

  if constexpr (!KREG) dma_tile<kTile, D, NT, SR>(sK, K, a.rk, tk0, a.nk, tid);
  dma_tile<kTile, D, NT, SR>(sV, V, a.rv, tk0, a.nk, tid);
  V8 kop[KREG ? 2 : 1][KC];
  if constexpr (KREG) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      load_operand_rows<D, E>(kop[mb], K + rrow<SR, D>(a.rk, min(tk0 + 32 * mb + (lane & 31), a.nk - 1)), true,
                              gq);
  }
  const int myr = wave * 32 + (lane & 31);  // this lane's query row in the tile
  const int myq = lt.tq0 + myr;
  const bool qvalid = lt.real(myr);
  V8 qop[KC];
  load_operand_rows<D, E>(qop, Q + rrow<SR, D>(a.rq, myq), qvalid, gq);
  __syncthreads();

  f32x16 s[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    s[mb] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      s[mb] = mfma32<E>(KREG ? kop[mb][kc] : lds_row8<D, E>(sK, mb * 32, lane & 31, kc, gq), qop[kc], s[mb]);
  }
  // one 64-key window of 64 rows, whole: nothing to mask
  const bool full = lw == 6 && lq == 6 && tk0 + kTile <= a.nk;
  const float sl2 = a.scale * kLog2e;
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = s[mb][e] * sl2;
      if (!full) {
        const int key = 32 * mb + 8 * (e >> 2) + 4 * gq + (e & 3);
        if (!lt.vis(myr, key)) x = -INFINITY;
      }
      s[mb][e] = x;
      mx = fmaxf(mx, x);
    }
  mx = max_halves(mx);
  const float mb2 = qvalid ? mx : 0.f;  // row max of the scaled scores, log2 units
  float l = 0.f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(s[mb][e] - mb2);
      s[mb][e] = p;
      l += p;
    }
  l = sum_halves(l);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
#pragma unroll
  for (int c = 0; c < kTile / 16; ++c) {
    const V8 pop = acc_chunk<E>(s[c >> 1], c & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      oacc[db] = mfma32<E>(lds_tr8<D, E>(sV, 16 * c, 32 * db, lane), pop, oacc[db]);
  }
  // O rows through LDS (sK, or sV with K in registers, is free once every
  // wave is past its products) so that the global stores are whole rows, 16
  // bytes per lane
  uint16_t* stage = KREG ? sV : sK;
  __syncthreads();
  acc_to_lds<D, E>(stage, myr, oacc, qvalid ? 1.f / l : 0.f, gq);
  if (qvalid && gq == 0) a.lse[(int64_t)bh * a.nq + myq] = (mb2 + log2f(l)) * kLn2;
  __syncthreads();
  uint16_t* O = (uint16_t*)a.o + rslice<SR, D>(a.ro, bh, a.H, a.nq);
  store_tile<QR, D, NT, SR>(O, a.ro, lt.tq0, lt.qend, stage, tid);
}

// ----------------------------------------------------------------- backward

// QR: query buffer rows; waves 0-1 own the tile's keys, the QR / 32 waves
// after them its query rows
// Three waves per SIMD (three workgroups per CU, which the LDS allows at
// d <= 96): the register budget that gives measured 7% over the compiler's
// own choice of two waves per SIMD.
template <typename E, int D, int QR, bool SR>
__global__ __launch_bounds__(128 + 2 * QR) __attribute__((amdgpu_waves_per_eu(3))) void bwd_local_kernel(BwdArgs a, int ntile, int lw, int lq) {
  using V8 = typename E::v8;
  constexpr int NT = 128 + 2 * QR, KE = tile_elems<kTile, D>(), QE = tile_elems<QR, D>();
  constexpr int KC = D / 16, DB = D / 32, QB = QR / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[QE];
  __shared__ __attribute__((aligned(16))) uint16_t sK[KE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[KE];
  __shared__ __attribute__((aligned(16))) uint16_t sG[QE];  // dO
  __shared__ __attribute__((aligned(16))) float sL[QR];     // lse * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[QR];     // D_i

  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);
  const int bh = blockIdx.x / ntile;
  const int tile = blockIdx.x % ntile;
  const LocalTile lt = local_tile(tile, a.nq, lw, lq);
  const int tk0 = lt.tk0;
  const uint16_t* Q = (const uint16_t*)a.q + rslice<SR, D>(a.rq, bh, a.H, a.nq);
  const uint16_t* K = (const uint16_t*)a.k + rslice<SR, D>(a.rk, bh, a.H, a.nk);
  const uint16_t* V = (const uint16_t*)a.v + rslice<SR, D>(a.rv, bh, a.H, a.nk);
  const uint16_t* dO = (const uint16_t*)a.dout + rslice<SR, D>(a.rdo, bh, a.H, a.nq);
  dma_tile<QR, D, NT, SR>(sQ, Q, a.rq, lt.tq0, lt.qend, tid);
  dma_tile<kTile, D, NT, SR>(sK, K, a.rk, tk0, a.nk, tid);
  dma_tile<kTile, D, NT, SR>(sV, V, a.rv, tk0, a.nk, tid);
  dma_tile<QR, D, NT, SR>(sG, dO, a.rdo, lt.tq0, lt.qend, tid);
  if (tid < QR) sL[tid] = lt.real(tid) ? a.lse[(int64_t)bh * a.nq + lt.tq0 + tid] * kLog2e : 0.f;
  __syncthreads();

  const float sl2 = a.scale * kLog2e;
  const bool full = lw == 6 && lq == 6 && tk0 + kTile <= a.nk;
  const bool dq_wave = wave >= 2;
  // this lane's key (dK/dV waves) or query row (dQ waves) in the tile
  const int own = 32 * (dq_wave ? wave - 2 : wave) + (lane & 31);

  // dK/dV waves: x[qt] = P, y[qt] = dP for query rows 32 qt + ..., lane = key.
  // dQ waves:    x[mb] = P^T, y[mb] = dP^T for keys 32 mb + ..., lane = query.
  static_assert(QB <= 2, "at most 64 query rows per tile");
  f32x16 x[2], y[2];
  f32x16 acc0[DB], acc1[DB];  // dK^T, dV^T (dK/dV waves) or dQ^T (dQ waves, acc0)
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    acc0[db] = f32x16{};
    acc1[db] = f32x16{};
  }

  if (dq_wave) {
    const float lse2 = sL[own];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      x[mb] = f32x16{};
      y[mb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        x[mb] = mfma32<E>(lds_row8<D, E>(sK, 32 * mb, lane & 31, kc, gq), lds_row8<D, E>(sQ, 0, own, kc, gq),
                       x[mb]);
        y[mb] = mfma32<E>(lds_row8<D, E>(sV, 32 * mb, lane & 31, kc, gq), lds_row8<D, E>(sG, 0, own, kc, gq),
                       y[mb]);
      }
    }
    float dsum = with_mask(!full, [&](auto masked) {
      float sum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float arg = fmaf(x[mb][e], sl2, -lse2);
          if constexpr (decltype(masked)::value) {
            const int key = 32 * mb + 8 * (e >> 2) + 4 * gq + (e & 3);
            arg = lt.vis(own, key) ? arg : -INFINITY;
          }
          const float p = fast_exp2(arg);
          x[mb][e] = p;
          sum = fmaf(p, y[mb][e], sum);
        }
      return sum;
    });
    dsum = sum_halves(dsum);
    if (gq == 0) sD[own] = dsum;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) x[mb][e] = x[mb][e] * (y[mb][e] - dsum);
  } else {
#pragma unroll
    for (int qt = 0; qt < QB; ++qt) {
      x[qt] = f32x16{};
      y[qt] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        x[qt] = mfma32<E>(lds_row8<D, E>(sQ, 32 * qt, lane & 31, kc, gq), lds_row8<D, E>(sK, 0, own, kc, gq),
                       x[qt]);
        y[qt] = mfma32<E>(lds_row8<D, E>(sG, 32 * qt, lane & 31, kc, gq), lds_row8<D, E>(sV, 0, own, kc, gq),
                       y[qt]);
      }
      with_mask(!full, [&](auto masked) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(&sL[32 * qt + 8 * i + 4 * gq]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 4 * i + j;
            float arg = fmaf(x[qt][e], sl2, -L4[j]);
            if constexpr (decltype(masked)::value)
              arg = lt.vis(32 * qt + 8 * i + 4 * gq + j, own) ? arg : -INFINITY;
            x[qt][e] = fast_exp2(arg);
          }
        }
      });
      // dV^T += dO^T P over this tile's 32 query rows
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const V8 pop = acc_chunk<E>(x[qt], c);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc1[db] = mfma32<E>(lds_tr8<D, E>(sG, 32 * qt + 16 * c, 32 * db, lane), pop, acc1[db]);
      }
    }
  }

  __syncthreads();  // sD complete

  if (dq_wave) {
    // dQ^T += K^T dS^T over the tile's 64 keys
#pragma unroll
    for (int c = 0; c < kTile / 16; ++c) {
      const V8 dsop = acc_chunk<E>(x[c >> 1], c & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc0[db] = mfma32<E>(lds_tr8<D, E>(sK, 16 * c, 32 * db, lane), dsop, acc0[db]);
    }
  } else {
#pragma unroll
    for (int qt = 0; qt < QB; ++qt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 D4 = *reinterpret_cast<const f32x4*>(&sD[32 * qt + 8 * i + 4 * gq]);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[qt][4 * i + j] *= (y[qt][4 * i + j] - D4[j]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const V8 dsop = acc_chunk<E>(x[qt], c);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc0[db] = mfma32<E>(lds_tr8<D, E>(sQ, 32 * qt + 16 * c, 32 * db, lane), dsop, acc0[db]);
      }
    }
  }
  __syncthreads();
  if (dq_wave) {
    acc_to_lds<D, E>(sQ, own, acc0, a.scale, gq);
  } else {
    acc_to_lds<D, E>(sK, own, acc0, a.scale, gq);
    acc_to_lds<D, E>(sV, own, acc1, 1.f, gq);
  }
  __syncthreads();
  store_tile<QR, D, NT, SR>((uint16_t*)a.dq + rslice<SR, D>(a.rdq, bh, a.H, a.nq), a.rdq, lt.tq0,
                            lt.qend, sQ, tid);
  store_tile<kTile, D, NT, SR>((uint16_t*)a.dk + rslice<SR, D>(a.rdk, bh, a.H, a.nk), a.rdk, tk0,
                               a.nk, sK, tid);
  store_tile<kTile, D, NT, SR>((uint16_t*)a.dv + rslice<SR, D>(a.rdv, bh, a.H, a.nk), a.rdv, tk0,
                               a.nk, sV, tid);
}

int log2_of(int w) {
  int s = 0;
  while ((1 << s) < w) ++s;
  return s;
}

// the tile geometry of a launch: log2 of both windows, tiles per (b, h)
struct LocalLaunch {
  int lw, lq, ntile;
  bool wide;  // more than 32 query rows per tile
};

LocalLaunch local_launch(const MaskGeom& g) {
  LocalLaunch l;
  l.lw = log2_of(g.window);
  l.lq = log2_of(g.window_q);
  l.ntile = (g.nk + kTile - 1) / kTile;
  l.wide = ((kTile >> l.lw) << l.lq) > 32;
  return l;
}

template <typename E, int D, bool SR>
int fwd_ds(const FwdArgs& a, hipStream_t s) {
  const LocalLaunch l = local_launch(a.mg);
  const dim3 grid((unsigned)((int64_t)l.ntile * a.B * a.H));
  if (l.wide)
    hipLaunchKernelGGL((fwd_local_kernel<E, D, 64, SR>), grid, dim3(128), 0, s, a, l.ntile, l.lw,
                       l.lq);
  else
    hipLaunchKernelGGL((fwd_local_kernel<E, D, 32, SR>), grid, dim3(64), 0, s, a, l.ntile, l.lw, l.lq);
  return (int)hipGetLastError();
}

template <typename E, int D, bool SR>
int bwd_ds(const BwdArgs& a, hipStream_t s) {
  const LocalLaunch l = local_launch(a.mg);
  const dim3 grid((unsigned)((int64_t)l.ntile * a.B * a.H));
  if (l.wide)
    hipLaunchKernelGGL((bwd_local_kernel<E, D, 64, SR>), grid, dim3(256), 0, s, a, l.ntile, l.lw,
                       l.lq);
  else
    hipLaunchKernelGGL((bwd_local_kernel<E, D, 32, SR>), grid, dim3(192), 0, s, a, l.ntile, l.lw,
                       l.lq);
  return (int)hipGetLastError();
}

template <typename E, int D>
int fwd_d(const FwdArgs& a, hipStream_t s) {
  return rows_plain(a, D) ? fwd_ds<E, D, false>(a, s) : fwd_ds<E, D, true>(a, s);
}

template <typename E, int D>
int bwd_d(const BwdArgs& a, hipStream_t s) {
  return rows_plain(a, D) ? bwd_ds<E, D, false>(a, s) : bwd_ds<E, D, true>(a, s);
}

template <typename E>
int fwd_e(const FwdArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return fwd_d<E, 64>(a, s);
    case 96: return fwd_d<E, 96>(a, s);
    case 128: return fwd_d<E, 128>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

template <typename E>
int bwd_e(const BwdArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return bwd_d<E, 64>(a, s);
    case 96: return bwd_d<E, 96>(a, s);
    case 128: return bwd_d<E, 128>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_fwd_16_local(const FwdArgs& a, bool f16, int d, hipStream_t s) {
  return f16 ? fwd_e<F16>(a, d, s) : fwd_e<Bf16>(a, d, s);
}

int launch_bwd_16_local(const BwdArgs& a, bool f16, int d, hipStream_t s) {
  return f16 ? bwd_e<F16>(a, d, s) : bwd_e<Bf16>(a, d, s);
}

}  // namespace attn
