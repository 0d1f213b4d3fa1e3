// attn_fp32.hip -- fp32 attention kernels (forward, row-sum pre-pass, dK/dV,
// dQ) on the vector ALUs.
//
// fp32 inputs carry a 1e-5 accuracy budget, which bf16 MFMA operands cannot
// meet, and the fp32 workloads are small exact-check cases; so this path uses
// plain fp32 FMAs.  A wave owns one row (a query row in the forward and dQ
// kernels, a key row in the dK/dV kernel); its four groups of 16 lanes split
// the row's visible range, taking kU consecutive keys (queries) in turn, each
// lane holding D/16 of the d entries; dot products reduce across a group with
// cross-lane xor shuffles, and the groups' partial results are combined at the
// end (shuffles across the groups).  The visible range of every row is the
// interval of attn_common.hpp, so fully masked keys are never visited.  The
// forward uses the online softmax (running max and sum, rescaling the
// accumulator) in natural-log units, per group, the groups' maxima and sums
// merged at the end; the backward recomputes P = exp(s - lse).
#include "attn_common.hpp"

namespace attn {

namespace {

constexpr int kGroup = 16;       // lanes per group
constexpr int kSplit = 4;        // groups per row (one wave)
constexpr int kRowsPerBlock = 4; // rows (waves) per 256-thread block
constexpr int kU = 4;            // consecutive keys (or queries) per group step

// sum over the four groups of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float split_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float split_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 8, kGroup);
  x += __shfl_xor(x, 4, kGroup);
  x += __shfl_xor(x, 2, kGroup);
  x += __shfl_xor(x, 1, kGroup);
  return x;
}

template <int D>
__device__ __forceinline__ void load_slice(float (&dst)[D / kGroup], const float* row, int li) {
#pragma unroll
  for (int e = 0; e < D / kGroup; ++e) dst[e] = row[li + kGroup * e];
}

template <int D>
__device__ __forceinline__ float dot_slice(const float (&x)[D / kGroup], const float* row, int li) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < D / kGroup; ++e) s = fmaf(x[e], row[li + kGroup * e], s);
  return group_sum(s);
}

template <int D>
__global__ __launch_bounds__(256) void fwd_fp32_kernel(FwdArgs a) {
  constexpr int E = D / kGroup;
  const int li = threadIdx.x & (kGroup - 1), gi = (threadIdx.x & 63) / kGroup;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / 64);
  const int64_t rows = (int64_t)a.B * a.H * a.nq;
  if (row >= rows) return;  // whole waves leave together
  const int bh = (int)(row / a.nq);
  const int i = (int)(row % a.nq);
  const float* K = (const float*)a.k + a.rk.slice(bh, a.H);
  const float* V = (const float*)a.v + a.rv.slice(bh, a.H);
  float q[E], acc[E];
  load_slice<D>(q, (const float*)a.q + a.rq.slice(bh, a.H) + a.rq.row(i), li);
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int lo = a.mg.row_lo(i), hi = a.mg.row_hi(i);
  // kU keys per step: their loads are independent and issued together, and
  // the running max moves once per step (keys past hi: index clamped, p = 0)
  for (int j = lo + gi * kU; j < hi; j += kSplit * kU) {
    float s[kU], vr[kU][E];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int jj = min(j + u, hi - 1);
      const float qk = a.scale * dot_slice<D>(q, K + a.rk.row(jj), li);  // every lane shuffles
      s[u] = j + u < hi ? qk : -INFINITY;
      load_slice<D>(vr[u], V + a.rv.row(jj), li);
    }
    float mnew = m;
#pragma unroll
    for (int u = 0; u < kU; ++u) mnew = fmaxf(mnew, s[u]);
    const float alpha = expf(m - mnew);   // m = -inf on the first keys -> 0
    float p[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) p[u] = expf(s[u] - mnew);   // -inf (past hi) -> 0
    l *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      l += p[u];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(p[u], vr[u][e], acc[e]);
    }
    m = mnew;
  }
  // merge the groups: rescale each to the largest running max, then sum
  const float mx = split_max(m);
  const float sc = m == -INFINITY ? 0.f : expf(m - mx);
  l = split_sum(l * sc);
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = split_sum(acc[e] * sc);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* O = (float*)a.o + a.ro.slice(bh, a.H) + a.ro.row(i);
  if (gi == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) O[li + kGroup * e] = acc[e] * inv;
    if (li == 0) a.lse[row] = l > 0.f ? mx + logf(l) : -INFINITY;
  }
}

constexpr int kDsumRowsPerBlock = 256 / kGroup;  // one group per row

template <int D>
__global__ __launch_bounds__(256) void dsum_fp32_kernel(BwdArgs a) {
  constexpr int E = D / kGroup;
  const int li = threadIdx.x & (kGroup - 1);
  const int64_t row = (int64_t)blockIdx.x * kDsumRowsPerBlock + (threadIdx.x / kGroup);
  if (row >= (int64_t)a.B * a.H * a.nq) return;
  const int bh = (int)(row / a.nq);
  const int i = (int)(row % a.nq);
  float x[E];
  load_slice<D>(x, (const float*)a.o + a.ro.slice(bh, a.H) + a.ro.row(i), li);
  const float s = dot_slice<D>(x, (const float*)a.dout + a.rdo.slice(bh, a.H) + a.rdo.row(i), li);
  if (li == 0) a.dsum[row] = s;
}

template <int D>
__global__ __launch_bounds__(256) void dq_fp32_kernel(BwdArgs a) {
  constexpr int E = D / kGroup;
  const int li = threadIdx.x & (kGroup - 1), gi = (threadIdx.x & 63) / kGroup;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / 64);
  const int64_t rows = (int64_t)a.B * a.H * a.nq;
  if (row >= rows) return;
  const int bh = (int)(row / a.nq);
  const int i = (int)(row % a.nq);
  const float* K = (const float*)a.k + a.rk.slice(bh, a.H);
  const float* V = (const float*)a.v + a.rv.slice(bh, a.H);
  float q[E], g[E], acc[E];
  load_slice<D>(q, (const float*)a.q + a.rq.slice(bh, a.H) + a.rq.row(i), li);
  load_slice<D>(g, (const float*)a.dout + a.rdo.slice(bh, a.H) + a.rdo.row(i), li);
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const float lse = a.lse[row], dsv = a.dsum[row];
  const int lo = a.mg.row_lo(i), hi = a.mg.row_hi(i);
  for (int j = lo + gi * kU; j < hi; j += kSplit * kU) {
    float kr[kU][E], ds[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int jj = min(j + u, hi - 1);
      load_slice<D>(kr[u], K + a.rk.row(jj), li);
      float qk = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) qk = fmaf(q[e], kr[u][e], qk);
      const float p = expf(a.scale * group_sum(qk) - lse);
      const float gv = dot_slice<D>(g, V + a.rv.row(jj), li);  // every lane shuffles
      ds[u] = j + u < hi ? p * (gv - dsv) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(ds[u], kr[u][e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = split_sum(acc[e]);
  float* dQ = (float*)a.dq + a.rdq.slice(bh, a.H) + a.rdq.row(i);
  if (gi == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) dQ[li + kGroup * e] = acc[e] * a.scale;
  }
}

template <int D>
__global__ __launch_bounds__(256) void dkdv_fp32_kernel(BwdArgs a) {
  constexpr int E = D / kGroup;
  const int li = threadIdx.x & (kGroup - 1), gi = (threadIdx.x & 63) / kGroup;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / 64);
  const int64_t rows = (int64_t)a.B * a.H * a.nk;
  if (row >= rows) return;
  const int bh = (int)(row / a.nk);
  const int j = (int)(row % a.nk);
  const float* Q = (const float*)a.q + a.rq.slice(bh, a.H);
  const float* dO = (const float*)a.dout + a.rdo.slice(bh, a.H);
  const float* LSE = a.lse + (int64_t)bh * a.nq;
  const float* DS = a.dsum + (int64_t)bh * a.nq;
  float k[E], v[E], dk[E], dv[E];
  load_slice<D>(k, (const float*)a.k + a.rk.slice(bh, a.H) + a.rk.row(j), li);
  load_slice<D>(v, (const float*)a.v + a.rv.slice(bh, a.H) + a.rv.row(j), li);
#pragma unroll
  for (int e = 0; e < E; ++e) dk[e] = dv[e] = 0.f;
  const int lo = a.mg.col_lo(j), hi = a.mg.col_hi(j);
  for (int i = lo + gi * kU; i < hi; i += kSplit * kU) {
    float qr[kU][E], gr[kU][E], p[kU], ds[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int ii = min(i + u, hi - 1);
      load_slice<D>(qr[u], Q + a.rq.row(ii), li);
      load_slice<D>(gr[u], dO + a.rdo.row(ii), li);
      float qk = 0.f, gv = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        qk = fmaf(k[e], qr[u][e], qk);
        gv = fmaf(v[e], gr[u][e], gv);
      }
      const bool in = i + u < hi;
      const float sq = group_sum(qk), sg = group_sum(gv);  // every lane shuffles
      p[u] = in ? expf(a.scale * sq - LSE[ii]) : 0.f;
      ds[u] = in ? p[u] * (sg - DS[ii]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dv[e] = fmaf(p[u], gr[u][e], dv[e]);
        dk[e] = fmaf(ds[u], qr[u][e], dk[e]);
      }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dk[e] = split_sum(dk[e]);
    dv[e] = split_sum(dv[e]);
  }
  float* dK = (float*)a.dk + a.rdk.slice(bh, a.H) + a.rdk.row(j);
  float* dV = (float*)a.dv + a.rdv.slice(bh, a.H) + a.rdv.row(j);
  if (gi == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      dK[li + kGroup * e] = dk[e] * a.scale;
      dV[li + kGroup * e] = dv[e];
    }
  }
}

inline unsigned blocks_for(int64_t rows, int per_block = kRowsPerBlock) {
  return (unsigned)((rows + per_block - 1) / per_block);
}

template <int D>
int fwd_d(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((fwd_fp32_kernel<D>), dim3(blocks_for((int64_t)a.B * a.H * a.nq)), dim3(256),
                     0, s, a);
  return (int)hipGetLastError();
}

template <int D>
int bwd_d(const BwdArgs& a, hipStream_t s, int passes) {
  const int64_t qrows = (int64_t)a.B * a.H * a.nq, krows = (int64_t)a.B * a.H * a.nk;
  int err = 0;
  if (passes & kPassRowSum) {
    hipLaunchKernelGGL((dsum_fp32_kernel<D>), dim3(blocks_for(qrows, kDsumRowsPerBlock)), dim3(256), 0, s, a);
    if ((err = (int)hipGetLastError())) return err;
  }
  if (passes & kPassDKDV) {
    hipLaunchKernelGGL((dkdv_fp32_kernel<D>), dim3(blocks_for(krows)), dim3(256), 0, s, a);
    if ((err = (int)hipGetLastError())) return err;
  }
  if (passes & kPassDQ) {
    hipLaunchKernelGGL((dq_fp32_kernel<D>), dim3(blocks_for(qrows)), dim3(256), 0, s, a);
    if ((err = (int)hipGetLastError())) return err;
  }
  return 0;
}

}  // namespace

int launch_fwd_fp32(const FwdArgs& a, int d, hipStream_t s) {
  switch (d) {
    case 64: return fwd_d<64>(a, s);
    case 96: return fwd_d<96>(a, s);
    case 128: return fwd_d<128>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

int launch_bwd_fp32(const BwdArgs& a, int d, hipStream_t s, int passes) {
  switch (d) {
    case 64: return bwd_d<64>(a, s, passes);
    case 96: return bwd_d<96>(a, s, passes);
    case 128: return bwd_d<128>(a, s, passes);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace attn
