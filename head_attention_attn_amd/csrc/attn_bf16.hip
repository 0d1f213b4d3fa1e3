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
// in base 2 with scale*log2(e) folded into the scores.  Key tiles outside a
// workgroup's visible range are never loaded; tiles a wave cannot see are
// skipped by that wave; only tiles that are not fully visible are masked.
//
// Backward ("IHA-CUDA", Repository Structure: preprocess (dPsum, lse), flash
// backward, postprocess dQaccum -> dQ), restructured as three deterministic
// passes with no atomics:
//   dsum:  D_i = sum_c dO[i][c] * O[i][c]                       (fp32)
//   dK/dV: workgroup per block of 32*NW keys; each wave owns 32 keys (lane
//          columns) and loops over the visible 32-query tiles in LDS:
//            S = Q K^T, dP = dO V^T, P = exp(S*scale - lse), dS = P*(dP - D)
//            dV^T += dO^T P,  dK^T += Q^T dS   (dO^T, Q^T by transpose reads)
//   dQ:    workgroup per block of 32*NW queries; loops over visible 64-key
//          tiles:  S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
#include "attn_common.hpp"
#include "bf16_tile.hpp"

namespace attn {

namespace {

// ------------------------------------------------------------------ forward

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void fwd_bf16_kernel(FwdArgs a, int nqt) {
  constexpr int NT = NW * 64, BM = 32 * NW, BN = 64, STR = D + 8;
  constexpr int KC = D / 16, DB = D / 32, SL = lds_slots(BN, D) * 8;
  // two named buffers (not one indexed array) so that the compiler can tell
  // the tile being read from the tile whose direct-to-LDS loads are in flight
  __shared__ __attribute__((aligned(16))) uint16_t sK0[SL];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[SL];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[SL];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[SL];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 5;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);  // longest causal rows first
  const MaskGeom mg = a.mg;
  const int i0 = qt * BM, i1 = min(i0 + BM, a.nq);

  const uint16_t* Q = (const uint16_t*)a.q + (int64_t)bh * a.nq * D;
  const uint16_t* K = (const uint16_t*)a.k + (int64_t)bh * a.nk * D;
  const uint16_t* V = (const uint16_t*)a.v + (int64_t)bh * a.nk * D;

  const int wa = i0 + wave * 32, wb = min(wa + 32, a.nq);
  const int myq = wa + (lane & 31);
  const bool qvalid = myq < a.nq;

  int lo, hi, wlo = 0, whi = 0;
  mg.key_range(i0, i1, &lo, &hi);
  if (wa < a.nq) mg.key_range(wa, wb, &wlo, &whi);
  const int rlo = qvalid ? mg.row_lo(myq) : 0;
  const int rhi = qvalid ? mg.row_hi(myq) : 0;
  const float sl2 = a.scale * kLog2e;
  const int t0 = (lo / BN) * BN;

  if (lo < hi) {
    dma_tile<BN, D, NT>(sK0, K, t0, a.nk, tid);
    dma_tile<BN, D, NT>(sV0, V, t0, a.nk, tid);
  }
  bf16x8 qop[KC];
  load_operand_rows<D>(qop, Q + (int64_t)myq * D, qvalid, gq);

  float m = -INFINITY, l = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  // one key tile [j0, j0 + BN) from LDS: scores, online softmax, O += P V
  auto tile = [&](const uint16_t* k_l, const uint16_t* v_l, int j0) {
    if (!(j0 < whi && j0 + BN > wlo)) return;
    const bool full = mg.tile_full(wa, wb, j0, j0 + BN);
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        s[mb] = mfma32(lds_read8(k_l + (mb * 32 + (lane & 31)) * STR + 16 * kc + 8 * gq),
                       qop[kc], s[mb]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = s[mb][e] * sl2;
        if (!full) {
          const int key = j0 + 32 * mb + 8 * (e >> 2) + 4 * gq + (e & 3);
          if (key < rlo || key >= rhi) x = -INFINITY;
        }
        s[mb][e] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, xor32(mx));
    const float mnew = fmaxf(m, mx);
    const float mu = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - mu);
    float rs = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(s[mb][e] - mu);
        s[mb][e] = p;
        rs += p;
      }
    rs += xor32(rs);
    l = l * alpha + rs;
    m = mnew;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int c = 0; c < BN / 16; ++c) {
      const bf16x8 pop = acc_chunk(s[c >> 1], c & 1);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = mfma32(lds_read_tr8(v_l, STR, 16 * c, 32 * db, lane), pop, oacc[db]);
    }
  };

  if (lo < hi) {
    __syncthreads();
    for (int j0 = t0; j0 < hi; j0 += 2 * BN) {
      if (j0 + BN < hi) {
        dma_tile<BN, D, NT>(sK1, K, j0 + BN, a.nk, tid);
        dma_tile<BN, D, NT>(sV1, V, j0 + BN, a.nk, tid);
      }
      tile(sK0, sV0, j0);
      __syncthreads();
      if (j0 + BN >= hi) break;
      if (j0 + 2 * BN < hi) {
        dma_tile<BN, D, NT>(sK0, K, j0 + 2 * BN, a.nk, tid);
        dma_tile<BN, D, NT>(sV0, V, j0 + 2 * BN, a.nk, tid);
      }
      tile(sK1, sV1, j0 + BN);
      __syncthreads();
    }
  }

  if (qvalid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    store_row_bf16<D>((uint16_t*)a.o + ((int64_t)bh * a.nq + myq) * D, oacc, inv, gq);
    if (gq == 0)
      a.lse[(int64_t)bh * a.nq + myq] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------- backward: row sums

template <int D>
__global__ __launch_bounds__(256) void dsum_bf16_kernel(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ dout,
                                                        float* __restrict__ dsum, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int li = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows && li < D / 8) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(o + row * D + 8 * li);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(dout + row * D + 8 * li);
#pragma unroll
    for (int s = 0; s < 8; ++s) acc += (float)x[s] * (float)y[s];
  }
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  if (row < rows && li == 0) dsum[row] = acc;
}

// ------------------------------------------------------- backward: dK / dV

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void dkdv_bf16_kernel(BwdArgs a, int nkt) {
  constexpr int NT = NW * 64, BK = 32 * NW, BQ = 32, STR = D + 8;
  constexpr int KC = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][BQ * STR];
  __shared__ __attribute__((aligned(16))) uint16_t sO[2][BQ * STR];
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];
  __shared__ __attribute__((aligned(16))) float sD[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 5;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int kt = (int)(blockIdx.x / BH);  // causal: low key tiles see the most queries
  const MaskGeom mg = a.mg;
  const int k0 = kt * BK, k1 = min(k0 + BK, a.nk);

  const uint16_t* Q = (const uint16_t*)a.q + (int64_t)bh * a.nq * D;
  const uint16_t* dO = (const uint16_t*)a.dout + (int64_t)bh * a.nq * D;
  const uint16_t* K = (const uint16_t*)a.k + (int64_t)bh * a.nk * D;
  const uint16_t* V = (const uint16_t*)a.v + (int64_t)bh * a.nk * D;
  const float* LSE = a.lse + (int64_t)bh * a.nq;
  const float* DS = a.dsum + (int64_t)bh * a.nq;

  const int wk0 = k0 + wave * 32, wk1 = min(wk0 + 32, a.nk);
  const int myk = wk0 + (lane & 31);
  const bool kvalid = myk < a.nk;

  bf16x8 kop[KC], vop[KC];
  load_operand_rows<D>(kop, K + (int64_t)myk * D, kvalid, gq);
  load_operand_rows<D>(vop, V + (int64_t)myk * D, kvalid, gq);

  int lo, hi, wlo = 0, whi = 0;
  mg.query_range(k0, k1, &lo, &hi);
  if (wk0 < a.nk) mg.query_range(wk0, wk1, &wlo, &whi);
  const int clo = kvalid ? mg.col_lo(myk) : 0;
  const int chi = kvalid ? mg.col_hi(myk) : 0;
  const float sl2 = a.scale * kLog2e;

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  if (lo < hi) {
    TileLoader<BQ, D, NT> qt, ot;
    float lreg = 0.f, dreg = 0.f;
    auto load_rowstats = [&](int r0) {
      if (tid < BQ) {
        const int r = r0 + tid;
        const float x = r < a.nq ? LSE[r] : 0.f;
        lreg = x * kLog2e;
        dreg = r < a.nq ? DS[r] : 0.f;
      }
    };
    const int t0 = (lo / BQ) * BQ;
    qt.load(Q, t0, a.nq, tid);
    ot.load(dO, t0, a.nq, tid);
    load_rowstats(t0);
    qt.store(sQ[0], STR, tid);
    ot.store(sO[0], STR, tid);
    if (tid < BQ) {
      sL[0][tid] = lreg;
      sD[0][tid] = dreg;
    }
    __syncthreads();
    int cur = 0;
    for (int i0 = t0; i0 < hi; i0 += BQ) {
      const bool has_next = i0 + BQ < hi;
      if (has_next) {
        qt.load(Q, i0 + BQ, a.nq, tid);
        ot.load(dO, i0 + BQ, a.nq, tid);
        load_rowstats(i0 + BQ);
      }
      if (i0 < whi && i0 + BQ > wlo) {
        const bool full = mg.tile_full(i0, i0 + BQ, wk0, wk1) && wk1 == wk0 + 32;
        const uint16_t* q_l = sQ[cur];
        const uint16_t* o_l = sO[cur];
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          s = mfma32(lds_read8(q_l + (lane & 31) * STR + 16 * kc + 8 * gq), kop[kc], s);
          dp = mfma32(lds_read8(o_l + (lane & 31) * STR + 16 * kc + 8 * gq), vop[kc], dp);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 L4 = *reinterpret_cast<const f32x4*>(&sL[cur][8 * i + 4 * gq]);
          const f32x4 D4 = *reinterpret_cast<const f32x4*>(&sD[cur][8 * i + 4 * gq]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 4 * i + j;
            const int qi = i0 + 8 * i + 4 * gq + j;
            const bool vis = full || (qi >= clo && qi < chi);
            const float p = vis ? fast_exp2(s[e] * sl2 - L4[j]) : 0.f;
            s[e] = p;
            dp[e] = p * (dp[e] - D4[j]);
          }
        }
#pragma unroll
        for (int c = 0; c < BQ / 16; ++c) {
          const bf16x8 pop = acc_chunk(s, c);
          const bf16x8 dsop = acc_chunk(dp, c);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            dvacc[db] = mfma32(lds_read_tr8(o_l, STR, 16 * c, 32 * db, lane), pop, dvacc[db]);
            dkacc[db] = mfma32(lds_read_tr8(q_l, STR, 16 * c, 32 * db, lane), dsop, dkacc[db]);
          }
        }
      }
      if (has_next) {
        qt.store(sQ[cur ^ 1], STR, tid);
        ot.store(sO[cur ^ 1], STR, tid);
        if (tid < BQ) {
          sL[cur ^ 1][tid] = lreg;
          sD[cur ^ 1][tid] = dreg;
        }
      }
      __syncthreads();
      cur ^= 1;
    }
  }

  if (kvalid) {
    store_row_bf16<D>((uint16_t*)a.dk + ((int64_t)bh * a.nk + myk) * D, dkacc, a.scale, gq);
    store_row_bf16<D>((uint16_t*)a.dv + ((int64_t)bh * a.nk + myk) * D, dvacc, 1.f, gq);
  }
}

// ------------------------------------------------------------ backward: dQ

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void dq_bf16_kernel(BwdArgs a, int nqt) {
  constexpr int NT = NW * 64, BM = 32 * NW, BN = 64, STR = D + 8;
  constexpr int KC = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * STR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * STR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, gq = lane >> 5;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);
  const MaskGeom mg = a.mg;
  const int i0 = qt * BM, i1 = min(i0 + BM, a.nq);

  const uint16_t* Q = (const uint16_t*)a.q + (int64_t)bh * a.nq * D;
  const uint16_t* dO = (const uint16_t*)a.dout + (int64_t)bh * a.nq * D;
  const uint16_t* K = (const uint16_t*)a.k + (int64_t)bh * a.nk * D;
  const uint16_t* V = (const uint16_t*)a.v + (int64_t)bh * a.nk * D;

  const int wa = i0 + wave * 32, wb = min(wa + 32, a.nq);
  const int myq = wa + (lane & 31);
  const bool qvalid = myq < a.nq;

  bf16x8 qop[KC], dop[KC];
  load_operand_rows<D>(qop, Q + (int64_t)myq * D, qvalid, gq);
  load_operand_rows<D>(dop, dO + (int64_t)myq * D, qvalid, gq);
  const float lse2 = qvalid ? a.lse[(int64_t)bh * a.nq + myq] * kLog2e : 0.f;
  const float dsv = qvalid ? a.dsum[(int64_t)bh * a.nq + myq] : 0.f;

  int lo, hi, wlo = 0, whi = 0;
  mg.key_range(i0, i1, &lo, &hi);
  if (wa < a.nq) mg.key_range(wa, wb, &wlo, &whi);
  const int rlo = qvalid ? mg.row_lo(myq) : 0;
  const int rhi = qvalid ? mg.row_hi(myq) : 0;
  const float sl2 = a.scale * kLog2e;

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  if (lo < hi) {
    TileLoader<BN, D, NT> kt, vt;
    const int t0 = (lo / BN) * BN;
    kt.load(K, t0, a.nk, tid);
    vt.load(V, t0, a.nk, tid);
    kt.store(sK[0], STR, tid);
    vt.store(sV[0], STR, tid);
    __syncthreads();
    int cur = 0;
    for (int j0 = t0; j0 < hi; j0 += BN) {
      const bool has_next = j0 + BN < hi;
      if (has_next) {
        kt.load(K, j0 + BN, a.nk, tid);
        vt.load(V, j0 + BN, a.nk, tid);
      }
      if (j0 < whi && j0 + BN > wlo) {
        const bool full = mg.tile_full(wa, wb, j0, j0 + BN);
        const uint16_t* k_l = sK[cur];
        const uint16_t* v_l = sV[cur];
        f32x16 s[2], dp[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          s[mb] = f32x16{};
          dp[mb] = f32x16{};
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) {
            s[mb] = mfma32(lds_read8(k_l + (mb * 32 + (lane & 31)) * STR + 16 * kc + 8 * gq),
                           qop[kc], s[mb]);
            dp[mb] = mfma32(lds_read8(v_l + (mb * 32 + (lane & 31)) * STR + 16 * kc + 8 * gq),
                            dop[kc], dp[mb]);
          }
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            bool vis = true;
            if (!full) {
              const int key = j0 + 32 * mb + 8 * (e >> 2) + 4 * gq + (e & 3);
              vis = key >= rlo && key < rhi;
            }
            const float p = vis ? fast_exp2(s[mb][e] * sl2 - lse2) : 0.f;
            s[mb][e] = p * (dp[mb][e] - dsv);
          }
#pragma unroll
        for (int c = 0; c < BN / 16; ++c) {
          const bf16x8 dsop = acc_chunk(s[c >> 1], c & 1);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            dqacc[db] = mfma32(lds_read_tr8(k_l, STR, 16 * c, 32 * db, lane), dsop, dqacc[db]);
        }
      }
      if (has_next) {
        kt.store(sK[cur ^ 1], STR, tid);
        vt.store(sV[cur ^ 1], STR, tid);
      }
      __syncthreads();
      cur ^= 1;
    }
  }

  if (qvalid)
    store_row_bf16<D>((uint16_t*)a.dq + ((int64_t)bh * a.nq + myq) * D, dqacc, a.scale, gq);
}

template <int D>
int launch_fwd_d(const FwdArgs& a, hipStream_t s) {
  constexpr int NW = 4, BM = 32 * NW;
  const int nqt = (a.nq + BM - 1) / BM;
  const int64_t grid = (int64_t)nqt * a.B * a.H;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s, a, nqt);
  return (int)hipGetLastError();
}

template <int D>
int launch_bwd_d(const BwdArgs& a, hipStream_t s, int passes) {
  constexpr int NW = 4;
  int err = 0;
  if (passes & kPassRowSum) {
    const int64_t rows = (int64_t)a.B * a.H * a.nq;
    hipLaunchKernelGGL((dsum_bf16_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                       s, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.dsum, rows);
    if ((err = (int)hipGetLastError())) return err;
  }
  if (passes & kPassDKDV) {
    const int nkt = (a.nk + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL((dkdv_bf16_kernel<D, NW>), dim3((unsigned)((int64_t)nkt * a.B * a.H)),
                       dim3(NW * 64), 0, s, a, nkt);
    if ((err = (int)hipGetLastError())) return err;
  }
  if (passes & kPassDQ) {
    const int nqt = (a.nq + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL((dq_bf16_kernel<D, NW>), dim3((unsigned)((int64_t)nqt * a.B * a.H)),
                       dim3(NW * 64), 0, s, a, nqt);
    if ((err = (int)hipGetLastError())) return err;
  }
  return 0;
}

}  // namespace

int launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t s) {
  if (a.mg.local64()) return launch_fwd_bf16_local(a, d, s);
  switch (d) {
    case 64: return launch_fwd_d<64>(a, s);
    case 96: return launch_fwd_d<96>(a, s);
    case 128: return launch_fwd_d<128>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

int launch_bwd_bf16(const BwdArgs& a, int d, hipStream_t s, int passes) {
  if (a.mg.local64()) {
    // one fused kernel writes dQ, dK and dV; it takes no partial pass set
    if (passes != kPassAll) return (int)hipErrorInvalidValue;
    return launch_bwd_bf16_local(a, d, s);
  }
  switch (d) {
    case 64: return launch_bwd_d<64>(a, s, passes);
    case 96: return launch_bwd_d<96>(a, s, passes);
    case 128: return launch_bwd_d<128>(a, s, passes);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace attn
