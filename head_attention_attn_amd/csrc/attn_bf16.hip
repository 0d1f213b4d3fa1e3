// attn_bf16.hip -- bf16 attention kernels for gfx950: forward, the backward
// row-sum pre-pass, the dK/dV pass and the dQ pass.
//
// Forward ("IHA-CUDA", Repository Structure: flash forward + online softmax):
// one workgroup of NW waves per (batch*head, block of 32*NW query rows); each
// wave owns 32 query rows, one per lane column, so every softmax statistic of
// a row lives in the two lanes l and l^32.  Scores are computed transposed,
//     S^T (keys x queries) = K Q^T,      O^T (d x queries) += V^T P^T,
// with bf16 MFMA 32x32x16 and fp32 accumulation: the Q^T operand stays in
// registers for the whole key loop, K and V tiles of 64 keys are staged in LDS
// (two buffers: the next tile's global loads are in flight while the current
// tile is consumed), K is read row-wise and V column-wise with the LDS
// transpose read.  P^T leaves the score accumulator directly as the bf16
// operand of the PV contraction (no LDS round trip).  The online softmax runs
// in base 2 with scale*log2(e) folded into the scores, and its running max
// moves only when a row's scores exceed it by more than 2^kSlack.  Key tiles
// outside a workgroup's visible range are never loaded; tiles a wave cannot
// see are skipped by that wave; only tiles that are not fully visible are
// masked.  Workgroups take (slice, tile) items in the order of tile_of().
//
// Backward ("IHA-CUDA", Repository Structure: preprocess (dPsum, lse), flash
// backward, postprocess dQaccum -> dQ), restructured as three deterministic
// passes with no atomics:
//   dsum:  D_i = sum_c dO[i][c] * O[i][c]                       (fp32)
//   dK/dV: workgroup per block of keys, looping over the visible query
//          tiles in LDS:
//            S = Q K^T, dP = dO V^T, P = exp(S*scale - lse), dS = P*(dP - D)
//            dV^T += dO^T P,  dK^T += Q^T dS   (dO^T, Q^T by transpose reads)
//   dQ:    workgroup per block of 32*NW queries; loops over visible 64-key
//          tiles:  S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
#include "attn_common.hpp"
#include "bf16_tile.hpp"

namespace attn {

namespace {

// ------------------------------------------------------------------ forward

constexpr float kSlack = 8.f;  // log2 of the largest unnormalised P

template <typename E, int D, int NW, int MODE, bool SR, bool SB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu((SB && D <= 96) ? 4 : 2))) void fwd_bf16_kernel(FwdArgs a, int nqt) {
  using V8 = typename E::v8;
  static_assert(NW == 4, "O staging assumes 4 waves (two 64-row tiles)");
  constexpr int NT = NW * 64, BM = 32 * NW, BN = 64, TE = tile_elems<BN, D>();
  constexpr int KC = D / 16, DB = D / 32;
  // two named buffers (not one indexed array) so that the compiler can tell
  // the tile being read from the tile whose direct-to-LDS loads are in flight.
  // With few keys per row (SB: Nk <= 256, at most four tiles) one buffer:
  // half the LDS lets more workgroups share a CU, and they hide each
  // other's tile loads better than a workgroup's own prefetch does
  // (measured on the N = 196 workload: 30 -> 26 us).  There, at d <= 96,
  // each tile is taken as two 32-key halves with an online-softmax update
  // each: half the score registers, so four waves per SIMD fit and all of
  // that workload's workgroups run at once (26.5 -> 23.7 us)
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[SB ? 8 : TE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[SB ? 8 : TE];

  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);
  const int BH = a.B * a.H;
  MaskGeom mg = a.mg;
  if (MODE != kAnyMask) mg.mode = MODE;  // compile-time mask mode: visibility folds to one case
  // longest causal rows first
  const TileId tix = tile_of(blockIdx.x, BH, nqt, mg.mode == kCausal, true);
  const int bh = tix.bh, qt = tix.t;
  const int i0 = qt * BM, i1 = min(i0 + BM, a.nq);

  const uint16_t* Q = (const uint16_t*)a.q + rslice<SR, D>(a.rq, bh, a.H, a.nq);
  const uint16_t* K = (const uint16_t*)a.k + rslice<SR, D>(a.rk, bh, a.H, a.nk);
  const uint16_t* V = (const uint16_t*)a.v + rslice<SR, D>(a.rv, bh, a.H, a.nk);

  const int wa = i0 + wave * 32, wb = min(wa + 32, a.nq);
  const int myq = wa + (lane & 31);
  const bool qvalid = myq < a.nq;

  int lo, hi, wlo = 0, whi = 0;
  mg.key_range(i0, i1, &lo, &hi);
  if (wa < a.nq) mg.key_range(wa, wb, &wlo, &whi);
  const int rlo = qvalid ? mg.row_lo(myq) : 0;
  const int rhi = qvalid ? mg.row_hi(myq) : 0;
  const float sl2 = a.scale * kLog2e;
  const int t0 = range_tile_row(lo, BN, 0);
  // K / V tile loads; the short-sequence half-tile path (128 registers)
  // computes its lane offsets per load instead of holding them
  DmaLanes<BN, D, NT> dl(tid);
  auto dma = [&](uint16_t* t_l, const uint16_t* src, const RowMap& rm, int r0) {
    if constexpr (SB && D <= 96)
      dma_tile<BN, D, NT, SR>(t_l, src, rm, r0, a.nk, tid);
    else
      dma_tile_lanes<BN, D, NT, SR>(t_l, src, rm, r0, a.nk, tid, dl.off);
  };

  if (lo < hi) {
    dma(sK0, K, a.rk, t0);
    dma(sV0, V, a.rv, t0);
  }
  V8 qop[KC];
  load_operand_rows<D, E>(qop, Q + rrow<SR, D>(a.rq, myq), qvalid, gq);

  float m = -INFINITY, l = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  // one key tile [j0, j0 + BN) from LDS: scores, online softmax, O += P V
  auto tile = [&](const uint16_t* k_l, const uint16_t* v_l, int j0) {
    if (!(wlo < whi && j0 < whi && j0 + BN > wlo)) return;
    const bool full = mg.tile_full(wa, wb, j0, j0 + BN);
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        s[mb] = mfma32<E>(lds_row8<D, E>(k_l, mb * 32, lane & 31, kc, gq), qop[kc], s[mb]);
    }
    // scaled scores relative to the running max m (log2 units), masked
    // entries -inf.  (per-element masking under a uniform test of `full`;
    // hoisting that test out of the loop or masking branch-free measured 5%
    // and 23% slower here)
    const float meff = m == -INFINITY ? 0.f : m;
    float mx = -INFINITY;
    with_mask(!full, [&](auto masked) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = fmaf(s[mb][e], sl2, -meff);
          if constexpr (decltype(masked)::value) {
            const int key = j0 + 32 * mb + 8 * (e >> 2) + 4 * gq + (e & 3);
            x = ((key >= rlo) & (key < rhi)) ? x : -INFINITY;
          }
          s[mb][e] = x;
          mx = fmaxf(mx, x);
        }
    });
    mx = max_halves(mx);
    // m moves only when a row's first visible score arrives or its scores
    // exceed m by more than 2^kSlack; otherwise P = 2^x stays below 2^kSlack
    // and O, l keep their scale.  One wave-uniform test per tile.
    const bool need = m == -INFINITY ? mx > -INFINITY : mx > kSlack;
    if (__any(need)) {
      const float sh = need ? mx : 0.f;
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(-sh);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mb][e] -= sh;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      if (need) m = meff + sh;
    }
    float rs = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(s[mb][e]);
        s[mb][e] = p;
        rs += p;
      }
    l += rs;
#pragma unroll
    for (int c = 0; c < BN / 16; ++c) {
      const V8 pop = acc_chunk<E>(s[c >> 1], c & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = mfma32<E>(lds_tr8<D, E>(v_l, 16 * c, 32 * db, lane), pop, oacc[db]);
    }
  };

  // the 32-key half mb of a staged tile, with its own online-softmax
  // update: half the score registers of a whole tile
  auto half_tile = [&](const uint16_t* k_l, const uint16_t* v_l, int j0, int mb) {
    const int h0 = j0 + 32 * mb;
    if (!(wlo < whi && h0 < whi && h0 + 32 > wlo)) return;
    const bool full = mg.tile_full(wa, wb, h0, h0 + 32);
    f32x16 sc = {};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      sc = mfma32<E>(lds_row8<D, E>(k_l, mb * 32, lane & 31, kc, gq), qop[kc], sc);
    const float meff = m == -INFINITY ? 0.f : m;
    float mx = -INFINITY;
    with_mask(!full, [&](auto masked) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = fmaf(sc[e], sl2, -meff);
        if constexpr (decltype(masked)::value) {
          const int key = h0 + 8 * (e >> 2) + 4 * gq + (e & 3);
          x = ((key >= rlo) & (key < rhi)) ? x : -INFINITY;
        }
        sc[e] = x;
        mx = fmaxf(mx, x);
      }
    });
    mx = max_halves(mx);
    const bool need = m == -INFINITY ? mx > -INFINITY : mx > kSlack;
    if (__any(need)) {
      const float sh = need ? mx : 0.f;
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(-sh);
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] -= sh;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      if (need) m = meff + sh;
    }
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(sc[e]);
      sc[e] = p;
      rs += p;
    }
    l += rs;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const V8 pop = acc_chunk<E>(sc, c2);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = mfma32<E>(lds_tr8<D, E>(v_l, 16 * (2 * mb + c2), 32 * db, lane), pop, oacc[db]);
    }
  };

  if (SB && lo < hi) {
    for (int j0 = t0; j0 < hi; j0 += BN) {
      if (j0 != t0) {
        dma(sK0, K, a.rk, j0);
        dma(sV0, V, a.rv, j0);
      }
      __syncthreads();
      if constexpr (D <= 96) {
        half_tile(sK0, sV0, j0, 0);
        half_tile(sK0, sV0, j0, 1);
      } else {
        tile(sK0, sV0, j0);
      }
      __syncthreads();
    }
  } else if (!SB && lo < hi) {
    __syncthreads();
    for (int j0 = t0; j0 < hi; j0 += 2 * BN) {
      if (j0 + BN < hi) {
        dma(sK1, K, a.rk, j0 + BN);
        dma(sV1, V, a.rv, j0 + BN);
      }
      tile(sK0, sV0, j0);
      __syncthreads();
      if (j0 + BN >= hi) break;
      if (j0 + 2 * BN < hi) {
        dma(sK0, K, a.rk, j0 + 2 * BN);
        dma(sV0, V, a.rv, j0 + 2 * BN);
      }
      tile(sK1, sV1, j0 + BN);
      __syncthreads();
    }
  }
  // each lane's l holds the sums of its half of the row's keys (the two
  // halves share m, so every rescale applied to both): combined once here
  l = sum_halves(l);
  // every wave is past its last LDS read here (each path above ends in a
  // barrier, and with no visible key no tile was loaded): O rows go through
  // sK0 (waves 0, 1) and sV0 (waves 2, 3) for whole-row 16-byte stores
  const float inv = l > 0.f ? 1.f / l : 0.f;
  acc_to_lds<D, E>(wave < 2 ? sK0 : sV0, 32 * (wave & 1) + (lane & 31), oacc, inv, gq);
  if (qvalid && gq == 0)
    a.lse[(int64_t)bh * a.nq + myq] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  __syncthreads();
  uint16_t* O = (uint16_t*)a.o + rslice<SR, D>(a.ro, bh, a.H, a.nq);
  store_tile<64, D, NT, SR>(O, a.ro, i0, a.nq, sK0, tid);
  store_tile<64, D, NT, SR>(O, a.ro, i0 + 64, a.nq, sV0, tid);
}

// ------------------------------------------------------- backward: row sums

// 16 rows of one (b, h) slice per workgroup, 16 lanes per row
template <typename E, int D, bool SR>
__global__ __launch_bounds__(256) void dsum_bf16_kernel(BwdArgs a, int nblk) {
  using V8 = typename E::v8;
  const int bh = blockIdx.x / nblk;
  const int row = (blockIdx.x % nblk) * 16 + (threadIdx.x >> 4);
  const int li = threadIdx.x & 15;
  float acc = 0.f;
  if (row < a.nq && li < D / 8) {
    const uint16_t* o =
        (const uint16_t*)a.o + rslice<SR, D>(a.ro, bh, a.H, a.nq) + rrow<SR, D>(a.ro, row);
    const uint16_t* g =
        (const uint16_t*)a.dout + rslice<SR, D>(a.rdo, bh, a.H, a.nq) + rrow<SR, D>(a.rdo, row);
    const V8 x = *reinterpret_cast<const V8*>(o + 8 * li);
    const V8 y = *reinterpret_cast<const V8*>(g + 8 * li);
#pragma unroll
    for (int s = 0; s < 8; ++s) acc += (float)x[s] * (float)y[s];
  }
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  if (row < a.nq && li == 0) a.dsum[(int64_t)bh * a.nq + row] = acc;
}

// ------------------------------------------------------- backward: dK / dV

// Tile shape of the dK/dV pass per head dimension: KB = 32-key blocks per
// wave, BQ = query rows per LDS tile, WPE = waves per SIMD the register
// budget is sized for.  At D = 128 each wave owns 64 keys (one LDS operand
// read feeds two MFMAs, and the two key blocks give the scheduler independent
// softmax / MFMA work to interleave) at one wave per SIMD; below that, 32
// keys per wave at two waves per SIMD.
template <int D>
struct DkdvShape {
  static constexpr int KB = 1;
  static constexpr int BQ = 64;
  static constexpr int WPE = D == 128 ? 1 : 2;
};

template <typename E, int D, int NW, int MODE, bool SR>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DkdvShape<D>::WPE))) void dkdv_bf16_kernel(BwdArgs a, int nkt) {
  using V8 = typename E::v8;
  static_assert(NW == 4, "dK/dV staging assumes 4 waves");
  constexpr int KB = DkdvShape<D>::KB, BQ = DkdvShape<D>::BQ;
  constexpr int NT = NW * 64, BK = 32 * KB * NW, TE = tile_elems<BQ, D>();
  constexpr int KC = D / 16, DB = D / 32, NH = BQ / 32;
  // Q and dO tiles of BQ query rows, two named buffers each; per buffer the
  // row statistics: [h*64 .. h*64+31] = lse, [h*64+32 .. h*64+63] = D of
  // rows 32h .. 32h+31
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sG0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sG1[TE];
  __shared__ __attribute__((aligned(16))) float sS0[2 * BQ];
  __shared__ __attribute__((aligned(16))) float sS1[2 * BQ];

  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);
  const int BH = a.B * a.H;
  MaskGeom mg = a.mg;
  if (MODE != kAnyMask) mg.mode = MODE;  // compile-time mask mode: visibility folds to one case
  // causal: low key tiles see the most queries
  const TileId tix = tile_of(blockIdx.x, BH, nkt, mg.mode == kCausal, false);
  const int bh = tix.bh, kt = tix.t;
  const int k0 = kt * BK, k1 = min(k0 + BK, a.nk);

  const uint16_t* Q = (const uint16_t*)a.q + rslice<SR, D>(a.rq, bh, a.H, a.nq);
  const uint16_t* dO = (const uint16_t*)a.dout + rslice<SR, D>(a.rdo, bh, a.H, a.nq);
  const uint16_t* K = (const uint16_t*)a.k + rslice<SR, D>(a.rk, bh, a.H, a.nk);
  const uint16_t* V = (const uint16_t*)a.v + rslice<SR, D>(a.rv, bh, a.H, a.nk);
  const float* LSE = a.lse + (int64_t)bh * a.nq;
  const float* DS = a.dsum + (int64_t)bh * a.nq;

  // this wave's keys [wk0, wk1): KB blocks of 32, lane l owns key 32 kb + l % 32
  const int wk0 = k0 + wave * 32 * KB, wk1 = min(wk0 + 32 * KB, a.nk);

  int lo, hi, wlo = 0, whi = 0;
  mg.query_range(k0, k1, &lo, &hi);
  if (wk0 < a.nk) mg.query_range(wk0, wk1, &wlo, &whi);
  const float sl2 = a.scale * kLog2e;
  const int t0 = range_tile_row(lo, BQ, 0);
  DmaLanes<BQ, D, NT> dl(tid);

  auto load = [&](uint16_t* q_l, uint16_t* g_l, float* s_l, int r0) {
    dma_tile_lanes<BQ, D, NT, SR>(q_l, Q, a.rq, r0, a.nq, tid, dl.off);
    dma_tile_lanes<BQ, D, NT, SR>(g_l, dO, a.rdo, r0, a.nq, tid, dl.off);
    if (wave < NH) dma_rows_f32x2(s_l + 64 * wave, LSE, DS, r0 + 32 * wave, a.nq, lane);
  };
  if (lo < hi) load(sQ0, sG0, sS0, t0);

  V8 kop[KB][KC], vop[KB][KC];
  int clo[KB], chi[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int myk = wk0 + 32 * kb + (lane & 31);
    const bool kvalid = myk < a.nk;
    load_operand_rows<D, E>(kop[kb], K + rrow<SR, D>(a.rk, myk), kvalid, gq);
    load_operand_rows<D, E>(vop[kb], V + rrow<SR, D>(a.rv, myk), kvalid, gq);
    clo[kb] = kvalid ? mg.col_lo(myk) : 0;
    chi[kb] = kvalid ? mg.col_hi(myk) : 0;
  }

  f32x16 dkacc[KB][DB], dvacc[KB][DB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dkacc[kb][db] = f32x16{};
      dvacc[kb][db] = f32x16{};
    }

  // one query tile from LDS, in 32-row parts: S, dP, P, dS for this wave's
  // key blocks, then dV^T += dO^T P and dK^T += Q^T dS (each transposed
  // operand read serves every key block)
  auto tile = [&](const uint16_t* q_l, const uint16_t* g_l, const float* s_l, int i0) {
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int ih = i0 + 32 * h;
      if (!(wlo < whi && ih < whi && ih + 32 > wlo)) continue;
      f32x16 s[KB], dp[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const V8 qr = lds_row8<D, E>(q_l, 32 * h, lane & 31, kc, gq);
        const V8 gr = lds_row8<D, E>(g_l, 32 * h, lane & 31, kc, gq);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          s[kb] = mfma32<E>(qr, kop[kb][kc], s[kb]);
          dp[kb] = mfma32<E>(gr, vop[kb][kc], dp[kb]);
        }
      }
      V8 pop[KB][2], dsop[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int bk0 = wk0 + 32 * kb;
        const bool full = bk0 + 32 <= a.nk && mg.tile_full(ih, ih + 32, bk0, bk0 + 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(&s_l[64 * h + 8 * i + 4 * gq]);
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(&s_l[64 * h + 32 + 8 * i + 4 * gq]);
          // (per-element form measured faster at d = 64, 96 than the
          // hoisted masked / unmasked instances used at d = 128)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 4 * i + j;
            const int qi = ih + 8 * i + 4 * gq + j;
            const bool vis = full || (qi >= clo[kb] && qi < chi[kb]);
            const float p = vis ? fast_exp2(fmaf(s[kb][e], sl2, -L4[j] * kLog2e)) : 0.f;
            s[kb][e] = p;
            dp[kb][e] = p * (dp[kb][e] - D4[j]);
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          pop[kb][c] = acc_chunk<E>(s[kb], c);
          dsop[kb][c] = acc_chunk<E>(dp[kb], c);
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const V8 gt = lds_tr8<D, E>(g_l, 32 * h + 16 * c, 32 * db, lane);
          const V8 qt = lds_tr8<D, E>(q_l, 32 * h + 16 * c, 32 * db, lane);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            dvacc[kb][db] = mfma32<E>(gt, pop[kb][c], dvacc[kb][db]);
            dkacc[kb][db] = mfma32<E>(qt, dsop[kb][c], dkacc[kb][db]);
          }
        }
    }
  };

  if (lo < hi) {
    __syncthreads();
    for (int i0 = t0; i0 < hi; i0 += 2 * BQ) {
      if (i0 + BQ < hi) load(sQ1, sG1, sS1, i0 + BQ);
      tile(sQ0, sG0, sS0, i0);
      __syncthreads();
      if (i0 + BQ >= hi) break;
      if (i0 + 2 * BQ < hi) load(sQ0, sG0, sS0, i0 + 2 * BQ);
      tile(sQ1, sG1, sS1, i0 + BQ);
      __syncthreads();
    }
  }
  // dK, then dV: rows go through the four BQ-row tile buffers (wave w's
  // 32 KB rows in buffer w when KB * 32 == BQ, else in half of buffer w / 2)
  // for whole-row 16-byte stores
  static_assert(KB * 32 * NW == 4 * BQ || KB * 32 * NW * 2 == 4 * BQ, "staging shape");
  auto bufs = [&](int i) { return i == 0 ? sQ0 : i == 1 ? sG0 : i == 2 ? sQ1 : sG1; };
  uint16_t* dK = (uint16_t*)a.dk + rslice<SR, D>(a.rdk, bh, a.H, a.nk);
  uint16_t* dV = (uint16_t*)a.dv + rslice<SR, D>(a.rdv, bh, a.H, a.nk);
  constexpr int WR = 32 * KB;                       // rows per wave
  constexpr int WPB = BQ / WR;                      // waves per buffer
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (pass) __syncthreads();
    uint16_t* mine = bufs(wave / WPB);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      acc_to_lds<D, E>(mine, (wave % WPB) * WR + 32 * kb + (lane & 31), pass ? dvacc[kb] : dkacc[kb],
                    pass ? 1.f : a.scale, gq);
    __syncthreads();
    uint16_t* dst = pass ? dV : dK;
    const RowMap& rdst = pass ? a.rdv : a.rdk;
#pragma unroll
    for (int b = 0; b < NW / WPB; ++b) store_tile<BQ, D, NT, SR>(dst, rdst, k0 + b * BQ, a.nk, bufs(b), tid);
  }
}

// dK/dV pass at D = 128: a workgroup of 12 waves (three per SIMD) for 128
// keys, in two roles working one query tile apart.
//   score waves 0..7: the two waves of key block kb = w / 2 hold its 32 K and
//     V rows as register operands, and wave w takes query rows 16 (w % 2) ..
//     + 15 of each 32-row Q / dO tile: the transposed products S^T = K Q^T
//     and dP^T = V dO^T as 16 x 16 blocks (v_mfma_f32_16x16x32; lane l:
//     query 16 (w % 2) + l % 16, keys 4 (l / 16) .. + 3 of each 16-key
//     half), P = exp(S*scale - lse) and dS = P (dP - D), rounded to E and
//     handed over as its rows of the key block's [query][key] P and dS tiles
//     (8-byte chunks swizzled by ds_tile_off), zeros where the key block
//     sees none of the tile; the score waves also load the Q / dO tiles and
//     the row statistics;
//   accumulate waves 8..11: wave 8 + m owns key blocks 2 (m / 2) and
//     2 (m / 2) + 1 (64 keys) and head-dim half m % 2: dV^T += dO^T P,
//     dK^T += Q^T dS with 32x32x16 products, dO^T, Q^T and the P, dS
//     operands from transpose reads, each dO^T / Q^T read feeding the
//     products of both key blocks; when the caller gave room, wave m also
//     writes 16-key chunk m % 2 of each visible dS block of its two key
//     blocks to the workspace, in the dQ pass's operand order.
// Splitting a key block's softmax arithmetic over two score waves halves the
// dependency chain each carries per step (one wave per key block carried the
// whole 32 x 32 tile before: 849 -> 781 us on the causal workload), with the
// same LDS operand traffic: a score wave reads only its 16 query rows, each
// read feeding the products of both key halves.  An accumulate wave over 64
// keys rather than 32 reads each step's dO^T / Q^T operands once for two key
// blocks: the accumulate waves' LDS reads per step fall from 104 to 72 KB
// (790 -> 777 us causal, 441 -> 433 us sliding window; its 128 accumulator
// registers set the three-waves-per-SIMD budget).  Q / dO tiles cycle through
// three named buffers (one being loaded, one read by the score waves, one by
// the accumulate waves), P / dS through three more.
template <typename E, int D, int MODE, bool SR>
__global__ __launch_bounds__(768) __attribute__((amdgpu_waves_per_eu(3))) void dkdv_k16_kernel(BwdArgs a, int nkt) {
  using V8 = typename E::v8;
  using V4 = typename E::v4;
  static_assert(D == 128, "16-key score waves: d = 128");
  constexpr int NS = 512, BK = 128, BQ = 32, TE = tile_elems<BQ, D>();
  constexpr int KS = D / 32, PE = 4 * 2 * 64 * 8;  // 4 blocks x 2 chunks x 64 lanes x 16 B
  // the staged Q / dO tiles are read by rows 16 at a time (the score waves'
  // B operands) and transposed (the accumulate waves): the chunk swizzle on
  // row bits 1, 2 keeps both conflict-free.  The epilogue reuses two of them
  // as staging in the default layout.
  constexpr int kQdSwz = 1;
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sG0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sG1[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sQ2[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sG2[TE];
  __shared__ __attribute__((aligned(16))) float sS0[64];  // lse * log2(e) of 32 rows, then D
  __shared__ __attribute__((aligned(16))) float sS1[64];
  __shared__ __attribute__((aligned(16))) float sS2[64];
  __shared__ __attribute__((aligned(16))) uint16_t sP0[PE];
  __shared__ __attribute__((aligned(16))) uint16_t sD0[PE];
  __shared__ __attribute__((aligned(16))) uint16_t sP1[PE];
  __shared__ __attribute__((aligned(16))) uint16_t sD1[PE];
  __shared__ __attribute__((aligned(16))) uint16_t sP2[PE];
  __shared__ __attribute__((aligned(16))) uint16_t sD2[PE];

  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);
  const int BH = a.B * a.H;
  MaskGeom mg = a.mg;
  if (MODE != kAnyMask) mg.mode = MODE;
  // causal: low key tiles see the most queries
  const TileId tix = tile_of(blockIdx.x, BH, nkt, mg.mode == kCausal, false);
  const int bh = tix.bh, kt = tix.t;
  const int k0 = kt * BK, k1 = min(k0 + BK, a.nk);
  const int kb = (wave & 7) >> 1;          // key block of this wave (either role)
  const int wk0 = k0 + 32 * kb, wk1 = min(wk0 + 32, a.nk);

  const uint16_t* Q = (const uint16_t*)a.q + rslice<SR, D>(a.rq, bh, a.H, a.nq);
  const uint16_t* dO = (const uint16_t*)a.dout + rslice<SR, D>(a.rdo, bh, a.H, a.nq);
  const float* LSE = a.lse + (int64_t)bh * a.nq;
  const float* DS = a.dsum + (int64_t)bh * a.nq;

  int lo, hi, wlo = 0, whi = 0;
  mg.query_range(k0, k1, &lo, &hi);
  if (wk0 < a.nk) mg.query_range(wk0, wk1, &wlo, &whi);
  const int t0 = range_tile_row(lo, BQ, 0);
  const int ntiles = lo < hi ? (hi - t0 + BQ - 1) / BQ : 0;
  // does this wave's key block see any row of tile j (an empty query range
  // [wlo, whi) sees none)
  auto sees = [&](int j) {
    const int i0 = t0 + j * BQ;
    return wlo < whi && i0 < whi && i0 + BQ > wlo;
  };

  if (wave < 8) {
    // ---------------------------------------------------------- score waves
    // Q / dO / lse / D of tile j are fetched into registers one step before
    // they are written to LDS (fetch(j + 3) is issued right after put(j + 2))
    RegTile<BQ, D, NS> rq, rg;
    float rstat = 0.f;
    auto fetch = [&](int j) {
      const int r0 = t0 + j * BQ;
      rq.template load<SR>(Q, a.rq, r0, a.nq, tid);
      rg.template load<SR>(dO, a.rdo, r0, a.nq, tid);
      // every lane loads (no branch around a load: a value loaded under a
      // divergent branch is waited for where the branch rejoins, which would
      // cancel the prefetch); only threads 0..63 store theirs
      const int t = tid & 63;
      rstat = (t < 32 ? LSE : DS)[min(r0 + (t & 31), a.nq - 1)];
    };
    // lane offsets, re-read each step (opaque to loop-invariant hoisting,
    // which would keep one address register per buffer set and read and
    // spill): this thread's 16 bytes of a staged tile, the B operand reads
    // (plus 32 ks per head-dim chunk) and the P / dS writes of key half kh
    const int qh = wave & 1;                 // query half of the tile: rows 16 qh .. + 15
    const int g4 = lane >> 4;                // key group: keys 4 g4 .. + 3 of a 16-key half
    const int r = 16 * qh + (lane & 15);     // this lane's tile row
    static_assert(BQ * D / 8 == NS, "one 16-byte piece of a staged tile per thread");
    int poff = toff<D, kQdSwz>(tid / (D / 8), (tid % (D / 8)) * 8);
    int roff = toff2<D, kQdSwz>(16 * qh, lane & 15, 0, 8 * g4);
    int woff[2] = {kb * 1024 + ds_tile_off(r, g4), kb * 1024 + ds_tile_off(r, 4 + g4)};
    int soff = tid;
    auto opaque = [&]() {
      asm volatile("" : "+v"(poff), "+v"(roff), "+v"(woff[0]), "+v"(woff[1]), "+v"(soff));
    };
    auto put = [&](uint16_t* q_l, uint16_t* g_l, float* s_l) {
      opaque();
      *reinterpret_cast<uint4*>(q_l + poff) = rq.r[0];
      *reinterpret_cast<uint4*>(g_l + poff) = rg.r[0];
      if (tid < 64) s_l[soff] = tid < 32 ? rstat * kLog2e : rstat;  // lse in log2 units
    };
    // put tile j into a set and fetch tile j + 1 into the registers
    auto load = [&](uint16_t* q_l, uint16_t* g_l, float* s_l, int j) {
      put(q_l, g_l, s_l);
      if (j + 1 < ntiles) fetch(j + 1);
    };
    if (ntiles > 0) {
      fetch(0);
      load(sQ0, sG0, sS0, 0);
    }
    if (ntiles > 1) load(sQ1, sG1, sS1, 1);

    const uint16_t* K = (const uint16_t*)a.k + rslice<SR, D>(a.rk, bh, a.H, a.nk);
    const uint16_t* V = (const uint16_t*)a.v + rslice<SR, D>(a.rv, bh, a.H, a.nk);
    // A operands (16 keys x 32 head dims per product): for key half kh, lane
    // l holds key wk0 + 16 kh + l % 16, dims 32 ks + 8 (l / 16) .. + 7
    V8 kop[2][KS], vop[2][KS];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int myk = wk0 + 16 * kh + (lane & 15);
      const bool kvalid = myk < a.nk;
      const uint16_t* kr = K + rrow<SR, D>(a.rk, kvalid ? myk : 0);
      const uint16_t* vr = V + rrow<SR, D>(a.rv, kvalid ? myk : 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kop[kh][ks] = kvalid ? *reinterpret_cast<const V8*>(kr + 32 * ks + 8 * g4) : V8{};
        vop[kh][ks] = kvalid ? *reinterpret_cast<const V8*>(vr + 32 * ks + 8 * g4) : V8{};
      }
    }
    const float sl2 = a.scale * kLog2e;

    auto produce = [&](const uint16_t* q_l, const uint16_t* g_l, const float* s_l,
                       uint16_t* p_l, uint16_t* d_l, int j) {
      opaque();
      if (!sees(j)) {
        // zeros: the accumulate wave of this key block's pair multiplies
        // both blocks' tiles whenever either block sees the tile
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          *reinterpret_cast<V4*>(p_l + woff[kh]) = V4{};
          *reinterpret_cast<V4*>(d_l + woff[kh]) = V4{};
        }
        return;
      }
      const int i0 = t0 + j * BQ;
      const bool full = wk1 == wk0 + 32 && mg.tile_full(i0 + 16 * qh, i0 + 16 * qh + 16, wk0, wk1);
      // read i: the B operand (32 dims x 16 queries) of head-dim chunk
      // i % 4, a row read of the Q (i < 4) or dO tile: lane l holds query
      // 16 qh + l % 16, dims 32 (i % 4) + 8 (l / 16) .. + 7; each read feeds
      // the products of both key halves.  Reads run kLead ahead.
      constexpr int NR = 2 * KS, kLead = 2;
      V8 op[NR];
      auto rd = [&](int i) {
        op[i] = *reinterpret_cast<const V8*>((i < KS ? q_l : g_l) + roff + 32 * (i % KS));
      };
      f32x4 s[2] = {f32x4{}, f32x4{}}, dp[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int i = 0; i < kLead; ++i) rd(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int ks = i % KS;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          if (i < KS)
            s[kh] = mfma16<E>(kop[kh][ks], op[i], s[kh]);
          else
            dp[kh] = mfma16<E>(vop[kh][ks], op[i], dp[kh]);
        }
        if (i + kLead < NR) rd(i + kLead);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float lq = s_l[r];       // lse * log2(e) of this lane's query
      const float dq = s_l[32 + r];  // D of this lane's query
      with_mask(!full, [&](auto masked) {
        // keys visible to this lane's query (none past the last row)
        const int qi = i0 + r;
        const int rlo = qi < a.nq ? mg.row_lo(qi) : 0, rhi = qi < a.nq ? mg.row_hi(qi) : 0;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float arg = fmaf(s[kh][e], sl2, -lq);
            if constexpr (decltype(masked)::value) {
              const int kj = wk0 + 16 * kh + 4 * g4 + e;
              arg = ((kj >= rlo) & (kj < rhi)) ? arg : -INFINITY;
            }
            s[kh][e] = fast_exp2(arg);
          }
      });
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[kh][e] = s[kh][e] * (dp[kh][e] - dq);
      // this lane's row of the [query][key] P and dS tiles of the key block
      // (ds_tile_off, 4-key chunk 4 kh + g4); the accumulate waves read them
      // transposed
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        *reinterpret_cast<V4*>(p_l + woff[kh]) = __builtin_convertvector(s[kh], V4);
        *reinterpret_cast<V4*>(d_l + woff[kh]) = __builtin_convertvector(dp[kh], V4);
      }
    };

    if (ntiles > 0) {
      __syncthreads();
      produce(sQ0, sG0, sS0, sP0, sD0, 0);
      __syncthreads();
    }
    // step j: load tile j + 2, produce tile j + 1 (the accumulate waves
    // consume tile j meanwhile), barrier
    for (int j = 0; j < ntiles; j += 3) {
      if (j + 2 < ntiles) load(sQ2, sG2, sS2, j + 2);
      produce(sQ1, sG1, sS1, sP1, sD1, j + 1);
      __syncthreads();
      if (j + 1 >= ntiles) break;
      if (j + 3 < ntiles) load(sQ0, sG0, sS0, j + 3);
      produce(sQ2, sG2, sS2, sP2, sD2, j + 2);
      __syncthreads();
      if (j + 2 >= ntiles) break;
      if (j + 4 < ntiles) load(sQ1, sG1, sS1, j + 4);
      produce(sQ0, sG0, sS0, sP0, sD0, j + 3);
      __syncthreads();
    }
    // staging barriers of the accumulate waves' epilogue
    __syncthreads();
    __syncthreads();
    __syncthreads();
  } else {
    // ----------------------------------------------------- accumulate waves
    // wave 8 + w: key blocks 2 kp and 2 kp + 1 (kp = w / 2, 64 keys), head
    // dims 64 dh .. + 63 (dh = w % 2)
    const int kp = (wave - 8) >> 1, dh = wave & 1;
    int trlo, trhi;           // lane offsets of the transposed reads, at dim 64 dh
    tr_lane_offsets<D, kQdSwz>(lane, trlo, trhi);
    trlo += 64 * dh;
    trhi += 64 * dh;
    int dso[2][2];            // lane offsets of the P / dS tile reads
    ds_tr_lane_offsets(lane, dso);
    // query range and first kept dS block of each of the two key blocks
    int blo[2] = {0, 0}, bhi[2] = {0, 0};
    int64_t bds[2] = {0, 0};
    uint16_t* dsb = a.ds;
    if (a.ds) dsb += (int64_t)bh * a.ds_per_bh * kDsBlockElems;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      const int bk0 = k0 + 32 * (2 * kp + b2);
      if (bk0 < a.nk) mg.query_range(bk0, min(bk0 + 32, a.nk), &blo[b2], &bhi[b2]);
      if (a.ds) {
        // every lane holds the total: keep it in scalar registers
        const int64_t v = ds_offset(mg, bk0 / 32, lane);
        const uint32_t vlo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t vhi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
        bds[b2] = (int64_t)(((uint64_t)vhi << 32) | vlo) - blo[b2] / 32;
      }
    }
    // kept-dS copy: this lane's two 8-byte reads of a dS tile and its 16
    // bytes of a block
    int cpo[2] = {ds_tile_off(lane & 31, 4 * dh + gq), ds_tile_off(lane & 31, 4 * dh + 2 + gq)};
    const int cpl = (dh * 64 + lane) * 8;
    auto seesb = [&](int j, int b2) {
      const int i0 = t0 + j * BQ;
      return blo[b2] < bhi[b2] && i0 < bhi[b2] && i0 + BQ > blo[b2];
    };
    f32x16 dkacc[2][2], dvacc[2][2];  // [key block][32-dim block]
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        dkacc[b2][db] = f32x16{};
        dvacc[b2][db] = f32x16{};
      }
    auto consume = [&](const uint16_t* q_l, const uint16_t* g_l, const uint16_t* p_l,
                       const uint16_t* d_l, int j) {
      if (!seesb(j, 0) && !seesb(j, 1)) return;
      const uint16_t* pt = p_l + 2 * kp * 1024;
      const uint16_t* dt = d_l + 2 * kp * 1024;
      // the lane offsets are re-read each step (opaque to loop-invariant
      // hoisting, which would keep one address register per read and buffer
      // set and spill)
      asm volatile("" : "+v"(trlo), "+v"(trhi), "+v"(dso[0][0]), "+v"(dso[0][1]), "+v"(dso[1][0]),
                   "+v"(dso[1][1]), "+v"(cpo[0]), "+v"(cpo[1]));
      // phase f = 2 c + kind: 16-row chunk c, dV (kind 0: dO^T x P) or dK
      // (kind 1: Q^T x dS); operands X[db] (dims 32 db of this wave's half)
      // and Y[b2] (key block 2 kp + b2); each X read feeds two products.
      // Read r of the 16: phase r / 4, X0 X1 Y0 Y1; issued one phase ahead
      constexpr int NR = 16;
      V8 rd[NR];
      auto issue = [&](int r) {
        const int f = r / 4, c = f / 2, kind = f % 2, q = r % 4;
        if (q < 2)
          rd[r] = lds_tr8_at<E>(kind ? q_l : g_l, trlo, trhi, 16 * c * tstride<D>() + 32 * q);
        else
          rd[r] = lds_tr8_ds_at<E>((kind ? dt : pt) + (q - 2) * 1024, dso[c]);
      };
#pragma unroll
      for (int r = 0; r < 4; ++r) issue(r);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int kind = f % 2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int db = k / 2, b2 = k % 2;
          const V8 x = rd[4 * f + db], y = rd[4 * f + 2 + b2];
          if (kind)
            dkacc[b2][db] = mfma32<E>(x, y, dkacc[b2][db]);
          else
            dvacc[b2][db] = mfma32<E>(x, y, dvacc[b2][db]);
          if (f < 3) issue(4 * (f + 1) + k);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (a.ds) {
        // keep chunk dh of each visible dS block for the dQ pass (block
        // i0 / 32 - blo / 32 of that key block's ds_count(); bds holds the
        // first block's index less blo / 32), in that pass's operand order
        // (lane l: query l % 32, keys 16 dh + 4 (l / 32) + 0..3 and
        // 16 dh + 8 + 4 (l / 32) + 0..3), streamed past the caches like the
        // output tiles
        const int i0 = t0 + j * BQ;
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
          if (!seesb(j, b2)) continue;
          const uint16_t* t = dt + b2 * 1024;
          const V4 x0 = *reinterpret_cast<const V4*>(t + cpo[0]);
          const V4 x1 = *reinterpret_cast<const V4*>(t + cpo[1]);
          uint16_t* blk = dsb + (bds[b2] + i0 / 32) * kDsBlockElems + cpl;
          __builtin_nontemporal_store(
              __builtin_bit_cast(u32x4, V8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]}),
              reinterpret_cast<u32x4*>(blk));
        }
      }
    };
    if (ntiles > 0) {
      __syncthreads();
      __syncthreads();
    }
    for (int j = 0; j < ntiles; j += 3) {
      consume(sQ0, sG0, sP0, sD0, j);
      __syncthreads();
      if (j + 1 >= ntiles) break;
      consume(sQ1, sG1, sP1, sD1, j + 1);
      __syncthreads();
      if (j + 2 >= ntiles) break;
      consume(sQ2, sG2, sP2, sD2, j + 2);
      __syncthreads();
    }
    // dK, then dV: key block kb's 32 rows through sQ0 / sG0 / sQ1 / sG1
    // (kb = 0 .. 3), each wave its two blocks' 64 dims
    uint16_t* m0 = kp == 0 ? sQ0 : sQ1;
    uint16_t* m1 = kp == 0 ? sG0 : sG1;
    constexpr int NA = 256;
    const int at = tid - NS;
    acc_to_lds_cols<D, E, 2>(m0, lane & 31, dkacc[0], 64 * dh, a.scale, gq);
    acc_to_lds_cols<D, E, 2>(m1, lane & 31, dkacc[1], 64 * dh, a.scale, gq);
    __syncthreads();
    uint16_t* dK = (uint16_t*)a.dk + rslice<SR, D>(a.rdk, bh, a.H, a.nk);
    store_tile<32, D, NA, SR>(dK, a.rdk, k0, a.nk, sQ0, at);
    store_tile<32, D, NA, SR>(dK, a.rdk, k0 + 32, a.nk, sG0, at);
    store_tile<32, D, NA, SR>(dK, a.rdk, k0 + 64, a.nk, sQ1, at);
    store_tile<32, D, NA, SR>(dK, a.rdk, k0 + 96, a.nk, sG1, at);
    __syncthreads();
    acc_to_lds_cols<D, E, 2>(m0, lane & 31, dvacc[0], 64 * dh, 1.f, gq);
    acc_to_lds_cols<D, E, 2>(m1, lane & 31, dvacc[1], 64 * dh, 1.f, gq);
    __syncthreads();
    uint16_t* dV = (uint16_t*)a.dv + rslice<SR, D>(a.rdv, bh, a.H, a.nk);
    store_tile<32, D, NA, SR>(dV, a.rdv, k0, a.nk, sQ0, at);
    store_tile<32, D, NA, SR>(dV, a.rdv, k0 + 32, a.nk, sG0, at);
    store_tile<32, D, NA, SR>(dV, a.rdv, k0 + 64, a.nk, sQ1, at);
    store_tile<32, D, NA, SR>(dV, a.rdv, k0 + 96, a.nk, sG1, at);
  }
}

// dQ pass from the kept dS blocks: dQ^T += K^T dS^T, nothing recomputed.
// Workgroup = 4 waves x 32 query rows; K tiles of 128 keys double-buffered in
// LDS (transpose reads give K^T), each wave's dS operands (16 bytes per lane
// per 16-key chunk, stored by the dK/dV pass in exactly this register order)
// loaded from the workspace one key tile ahead.
template <typename E, int D, int MODE, bool SR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void dq_ds_kernel(BwdArgs a, int nqt) {
  using V8 = typename E::v8;
  constexpr int NT = 256, BM = 128, BN = 128, TE = tile_elems<BN, D>();
  constexpr int DB = D / 32, NKB = BN / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TE];

  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);
  const int BH = a.B * a.H;
  MaskGeom mg = a.mg;
  if (MODE != kAnyMask) mg.mode = MODE;
  // longest causal rows first
  const TileId tix = tile_of(blockIdx.x, BH, nqt, mg.mode == kCausal, true);
  const int bh = tix.bh, qt = tix.t;
  const int i0 = qt * BM, i1 = min(i0 + BM, a.nq);
  const uint16_t* K = (const uint16_t*)a.k + rslice<SR, D>(a.rk, bh, a.H, a.nk);
  const uint16_t* DS = a.ds + (int64_t)bh * a.ds_per_bh * kDsBlockElems;

  const int wa = i0 + wave * 32;
  const int jq = wa / 32;  // this wave's query block
  int lo, hi;
  mg.key_range(i0, i1, &lo, &hi);
  const int t0 = range_tile_row(lo, BN, 0);
  DmaLanes<BN, D, NT> dl(tid);

  // running block cursor: index of key block `kbn`'s first dS block
  int kbn = t0 / 32;
  int64_t cur = lo < hi ? ds_offset(mg, kbn, lane) : 0;
  // operands of the 4 key blocks of one tile; bit kb of the mask: block kb
  // has this wave's query block
  auto fetch = [&](V8 (&op)[NKB][2], unsigned& valid) {
    valid = 0;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int jlo = mg.ds_jlo(kbn), cnt = mg.ds_count(kbn);
      if (wa < a.nq && jq >= jlo && jq < jlo + cnt) {
        const uint16_t* blk = DS + (cur + (jq - jlo)) * kDsBlockElems;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          op[kb][cc] = *reinterpret_cast<const V8*>(blk + (cc * 64 + lane) * 8);
        valid |= 1u << kb;
      }
      cur += cnt;
      ++kbn;
    }
  };

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};
  auto tile = [&](const uint16_t* k_l, const V8 (&op)[NKB][2], unsigned valid) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (!(valid & (1u << kb))) continue;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dqacc[db] = mfma32<E>(lds_tr8<D, E>(k_l, 32 * kb + 16 * cc, 32 * db, lane), op[kb][cc], dqacc[db]);
    }
  };

  if (lo < hi) {
    V8 opA[NKB][2], opB[NKB][2];
    unsigned vA = 0, vB = 0;
    dma_tile_lanes<BN, D, NT, SR>(sK0, K, a.rk, t0, a.nk, tid, dl.off);
    fetch(opA, vA);
    __syncthreads();
    for (int j0 = t0; j0 < hi; j0 += 2 * BN) {
      if (j0 + BN < hi) {
        dma_tile_lanes<BN, D, NT, SR>(sK1, K, a.rk, j0 + BN, a.nk, tid, dl.off);
        fetch(opB, vB);
      }
      tile(sK0, opA, vA);
      __syncthreads();
      if (j0 + BN >= hi) break;
      if (j0 + 2 * BN < hi) {
        dma_tile_lanes<BN, D, NT, SR>(sK0, K, a.rk, j0 + 2 * BN, a.nk, tid, dl.off);
        fetch(opA, vA);
      }
      tile(sK1, opB, vB);
      __syncthreads();
    }
  }
  acc_to_lds<D, E>(sK0, 32 * wave + (lane & 31), dqacc, a.scale, gq);
  __syncthreads();
  store_tile<BM, D, NT, SR>((uint16_t*)a.dq + rslice<SR, D>(a.rdq, bh, a.H, a.nq), a.rdq, i0, a.nq,
                            sK0, tid);
}

// ------------------------------------------------------------ backward: dQ

template <typename E, int D, int NW, int MODE, bool SR>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void dq_bf16_kernel(BwdArgs a, int nqt) {
  using V8 = typename E::v8;
  static_assert(NW == 4, "dQ staging assumes 4 waves (two 64-row tiles)");
  constexpr int NT = NW * 64, BM = 32 * NW, BN = 64, TE = tile_elems<BN, D>();
  constexpr int KC = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TE];

  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 5;
  const int wave = wave_id(tid);
  const int BH = a.B * a.H;
  MaskGeom mg = a.mg;
  if (MODE != kAnyMask) mg.mode = MODE;  // compile-time mask mode: visibility folds to one case
  // longest causal rows first
  const TileId tix = tile_of(blockIdx.x, BH, nqt, mg.mode == kCausal, true);
  const int bh = tix.bh, qt = tix.t;
  const int i0 = qt * BM, i1 = min(i0 + BM, a.nq);

  const uint16_t* Q = (const uint16_t*)a.q + rslice<SR, D>(a.rq, bh, a.H, a.nq);
  const uint16_t* dO = (const uint16_t*)a.dout + rslice<SR, D>(a.rdo, bh, a.H, a.nq);
  const uint16_t* K = (const uint16_t*)a.k + rslice<SR, D>(a.rk, bh, a.H, a.nk);
  const uint16_t* V = (const uint16_t*)a.v + rslice<SR, D>(a.rv, bh, a.H, a.nk);

  const int wa = i0 + wave * 32, wb = min(wa + 32, a.nq);
  const int myq = wa + (lane & 31);
  const bool qvalid = myq < a.nq;

  int lo, hi, wlo = 0, whi = 0;
  mg.key_range(i0, i1, &lo, &hi);
  if (wa < a.nq) mg.key_range(wa, wb, &wlo, &whi);
  const int rlo = qvalid ? mg.row_lo(myq) : 0;
  const int rhi = qvalid ? mg.row_hi(myq) : 0;
  const float sl2 = a.scale * kLog2e;
  const int t0 = range_tile_row(lo, BN, 0);
  DmaLanes<BN, D, NT> dl(tid);

  if (lo < hi) {
    dma_tile_lanes<BN, D, NT, SR>(sK0, K, a.rk, t0, a.nk, tid, dl.off);
    dma_tile_lanes<BN, D, NT, SR>(sV0, V, a.rv, t0, a.nk, tid, dl.off);
  }
  V8 qop[KC], dop[KC];
  load_operand_rows<D, E>(qop, Q + rrow<SR, D>(a.rq, myq), qvalid, gq);
  load_operand_rows<D, E>(dop, dO + rrow<SR, D>(a.rdo, myq), qvalid, gq);
  const float lse2 = qvalid ? a.lse[(int64_t)bh * a.nq + myq] * kLog2e : 0.f;
  const float dsv = qvalid ? a.dsum[(int64_t)bh * a.nq + myq] : 0.f;

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  // one key tile [j0, j0 + BN): S^T, dP^T, dS^T per 32-key half (packed to
  // bf16 right away to keep the live set small), then dQ^T += K^T dS^T
  auto tile = [&](const uint16_t* k_l, const uint16_t* v_l, int j0) {
    if (!(wlo < whi && j0 < whi && j0 + BN > wlo)) return;
    const bool full = mg.tile_full(wa, wb, j0, j0 + BN);
    V8 dsop[BN / 16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        s = mfma32<E>(lds_row8<D, E>(k_l, mb * 32, lane & 31, kc, gq), qop[kc], s);
        dp = mfma32<E>(lds_row8<D, E>(v_l, mb * 32, lane & 31, kc, gq), dop[kc], dp);
      }
      with_mask(!full, [&](auto masked) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float arg = s[e] * sl2 - lse2;
          if constexpr (decltype(masked)::value) {
            const int key = j0 + 32 * mb + 8 * (e >> 2) + 4 * gq + (e & 3);
            arg = ((key >= rlo) & (key < rhi)) ? arg : -INFINITY;
          }
          s[e] = fast_exp2(arg) * (dp[e] - dsv);
        }
      });
      dsop[2 * mb] = acc_chunk<E>(s, 0);
      dsop[2 * mb + 1] = acc_chunk<E>(s, 1);
    }
#pragma unroll
    for (int c = 0; c < BN / 16; ++c)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        dqacc[db] = mfma32<E>(lds_tr8<D, E>(k_l, 16 * c, 32 * db, lane), dsop[c], dqacc[db]);
  };

  if (lo < hi) {
    __syncthreads();
    for (int j0 = t0; j0 < hi; j0 += 2 * BN) {
      if (j0 + BN < hi) {
        dma_tile_lanes<BN, D, NT, SR>(sK1, K, a.rk, j0 + BN, a.nk, tid, dl.off);
        dma_tile_lanes<BN, D, NT, SR>(sV1, V, a.rv, j0 + BN, a.nk, tid, dl.off);
      }
      tile(sK0, sV0, j0);
      __syncthreads();
      if (j0 + BN >= hi) break;
      if (j0 + 2 * BN < hi) {
        dma_tile_lanes<BN, D, NT, SR>(sK0, K, a.rk, j0 + 2 * BN, a.nk, tid, dl.off);
        dma_tile_lanes<BN, D, NT, SR>(sV0, V, a.rv, j0 + 2 * BN, a.nk, tid, dl.off);
      }
      tile(sK1, sV1, j0 + BN);
      __syncthreads();
    }
  }
  acc_to_lds<D, E>(wave < 2 ? sK0 : sV0, 32 * (wave & 1) + (lane & 31), dqacc, a.scale, gq);
  __syncthreads();
  uint16_t* dQ = (uint16_t*)a.dq + rslice<SR, D>(a.rdq, bh, a.H, a.nq);
  store_tile<64, D, NT, SR>(dQ, a.rdq, i0, a.nq, sK0, tid);
  store_tile<64, D, NT, SR>(dQ, a.rdq, i0 + 64, a.nq, sV0, tid);
}

template <typename E, int D, int MODE, bool SR>
int launch_fwd_dm(const FwdArgs& a, hipStream_t s) {
  constexpr int NW = 4, BM = 32 * NW;
  const int nqt = (a.nq + BM - 1) / BM;
  const int64_t grid = (int64_t)nqt * a.B * a.H;
  if (a.nk <= 256)
    hipLaunchKernelGGL((fwd_bf16_kernel<E, D, NW, kAnyMask, SR, true>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, s, a, nqt);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<E, D, NW, kAnyMask, SR, false>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, s, a, nqt);
  return (int)hipGetLastError();
}

template <typename E, int D, int MODE, bool SR>
int launch_bwd_dm(const BwdArgs& a, hipStream_t s, int passes) {
  constexpr int NW = 4;
  int err = 0;
  if (passes & kPassRowSum) {
    const int nblk = (a.nq + 15) / 16;
    hipLaunchKernelGGL((dsum_bf16_kernel<E, D, SR>), dim3((unsigned)((int64_t)nblk * a.B * a.H)),
                       dim3(256), 0, s, a, nblk);
    if ((err = (int)hipGetLastError())) return err;
  }
  if (passes & kPassDKDV) {
    if constexpr (D == 128) {
      const int nkt = (a.nk + 127) / 128;
      hipLaunchKernelGGL((dkdv_k16_kernel<E, D, kAnyMask, SR>),
                         dim3((unsigned)((int64_t)nkt * a.B * a.H)), dim3(768), 0, s, a, nkt);
    } else {
      constexpr int BK = 32 * DkdvShape<D>::KB * NW;
      const int nkt = (a.nk + BK - 1) / BK;
      hipLaunchKernelGGL((dkdv_bf16_kernel<E, D, NW, kAnyMask, SR>),
                         dim3((unsigned)((int64_t)nkt * a.B * a.H)), dim3(NW * 64), 0, s, a, nkt);
    }
    if ((err = (int)hipGetLastError())) return err;
  }
  if (passes & kPassDQ) {
    const int nqt = (a.nq + 32 * NW - 1) / (32 * NW);
    bool done = false;
    if constexpr (D == 128) {
      if (a.ds) {
        hipLaunchKernelGGL((dq_ds_kernel<E, D, MODE, SR>), dim3((unsigned)((int64_t)nqt * a.B * a.H)),
                           dim3(256), 0, s, a, nqt);
        done = true;
      }
    }
    if (!done)
      hipLaunchKernelGGL((dq_bf16_kernel<E, D, NW, MODE, SR>),
                         dim3((unsigned)((int64_t)nqt * a.B * a.H)), dim3(NW * 64), 0, s, a, nqt);
    if ((err = (int)hipGetLastError())) return err;
  }
  return 0;
}

template <typename E, int D>
int launch_fwd_d(const FwdArgs& a, hipStream_t s) {
  if (rows_plain(a, D)) return launch_fwd_dm<E, D, kAnyMask, false>(a, s);
  return launch_fwd_dm<E, D, kAnyMask, true>(a, s);
}

// The dQ kernel is instantiated per mask mode (measured 16% faster on the
// causal and sliding workloads with the visibility tests folded); the forward
// and dK/dV kernels read the mode at run time (their per-mode instances
// measured 3-4% slower on the causal workload).  Every kernel comes in a
// contiguous-rows and a strided-rows instance.
template <typename E, int D, bool SR>
int launch_bwd_ds(const BwdArgs& a, hipStream_t s, int passes) {
  switch (a.mg.mode) {
    case kNone: return launch_bwd_dm<E, D, kNone, SR>(a, s, passes);
    case kCausal: return launch_bwd_dm<E, D, kCausal, SR>(a, s, passes);
    case kSliding: return launch_bwd_dm<E, D, kSliding, SR>(a, s, passes);
    case kBlock: return launch_bwd_dm<E, D, kBlock, SR>(a, s, passes);
  }
  return (int)hipErrorInvalidValue;
}

template <typename E, int D>
int launch_bwd_d(const BwdArgs& a, hipStream_t s, int passes) {
  return rows_plain(a, D) ? launch_bwd_ds<E, D, false>(a, s, passes)
                          : launch_bwd_ds<E, D, true>(a, s, passes);
}

template <typename E>
int launch_fwd_e(const FwdArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_fwd_d<E, 64>(a, s);
    case 96: return launch_fwd_d<E, 96>(a, s);
    case 128: return launch_fwd_d<E, 128>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

template <typename E>
int launch_bwd_e(const BwdArgs& a, int d, hipStream_t s, int passes) {
  switch (d) {
    case 64: return launch_bwd_d<E, 64>(a, s, passes);
    case 96: return launch_bwd_d<E, 96>(a, s, passes);
    case 128: return launch_bwd_d<E, 128>(a, s, passes);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_fwd_16(const FwdArgs& a, bool f16, int d, hipStream_t s) {
  if (a.mg.local64()) return launch_fwd_16_local(a, f16, d, s);
  return f16 ? launch_fwd_e<F16>(a, d, s) : launch_fwd_e<Bf16>(a, d, s);
}

int launch_bwd_16(const BwdArgs& a, bool f16, int d, hipStream_t s, int passes) {
  if (a.mg.local64()) {
    // one fused kernel writes dQ, dK and dV; it takes no partial pass set
    if (passes != kPassAll) return (int)hipErrorInvalidValue;
    return launch_bwd_16_local(a, f16, d, s);
  }
  // every key of a (b, h) in one workgroup: the whole backward is one fused
  // kernel; a partial pass set runs the general passes
  if (passes == kPassAll && short_keys(a.mg, d)) return launch_bwd_16_short(a, f16, d, s);
  return f16 ? launch_bwd_e<F16>(a, d, s, passes) : launch_bwd_e<Bf16>(a, d, s, passes);
}

}  // namespace attn
