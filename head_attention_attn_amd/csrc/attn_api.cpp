// attn_api.cpp -- the C ABI of include/attn.h: argument validation, device
// gating and dispatch to the kernel launchers.  No device memory is allocated
// here and no state is kept per call; the global state is a per-device cache
// of "is this a gfx950" and, for attn_bwd_noalloc, a static device scratch
// array with a per-device cache of its address, both filled once under a
// mutex.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "attn_common.hpp"

static_assert(int(ATTN_PASS_ROWSUM) == int(attn::kPassRowSum) &&
                  int(ATTN_PASS_DKDV) == int(attn::kPassDKDV) &&
                  int(ATTN_PASS_DQ) == int(attn::kPassDQ) && int(ATTN_PASS_ALL) == int(attn::kPassAll),
              "pass bits of attn.h and the launchers agree");

// Scratch of attn_bwd_noalloc: device memory that the library holds (one
// copy per GPU, until the process ends) for callers that cannot allocate.  In
// host code `scratch` names a host-side stand-in, not the device array: host
// code uses only the device address that scratch_ptr() looks up.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxSeq = int64_t(1) << 30;   // per-(b,h) row counts fit int32 math
constexpr int64_t kMaxGrid = INT_MAX;           // 1-D grid of workgroups

bool supported_d(int64_t d) { return d == 64 || d == 96 || d == 128; }

size_t elem_size(int dtype) { return dtype == ATTN_FP32 ? 4 : 2; }

// bf16 and fp16 share the 16-bit kernels (MFMA with fp32 accumulation)
bool is16(int dtype) { return dtype == ATTN_BF16 || dtype == ATTN_FP16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common checks of sizes, dtype, d, mask and window.
int check_geometry(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   float scale, int mask, int64_t window) {
  if (!is16(dtype) && dtype != ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
  if (Nq > kMaxSeq || Nk > kMaxSeq || B * H > kMaxGrid) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  switch (mask) {
    case ATTN_MASK_NONE:
    case ATTN_MASK_CAUSAL:
      break;
    case ATTN_MASK_SLIDING:
      if (window < 1 || window > kMaxSeq) return ATTN_ERR_INVALID_ARG;
      break;
    case ATTN_MASK_BLOCK:
      // Nk / window windows of `window` keys; each holds Nq / (Nk / window)
      // query rows (fewer than `window` when queries are pooled)
      if (window < 1 || window > Nk || Nk % window != 0) return ATTN_ERR_INVALID_ARG;
      if (Nq % (Nk / window) != 0) return ATTN_ERR_INVALID_ARG;
      break;
    default:
      return ATTN_ERR_INVALID_ARG;
  }
  // the kernels' grids: at most INT_MAX workgroups of 16 rows
  const int64_t rowblocks = (std::max(Nq, Nk) + 15) / 16;
  if (B * H * rowblocks > kMaxGrid) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

size_t ws_size(int64_t B, int64_t H, int64_t Nq) {
  if (B < 1 || H < 1 || Nq < 1) return 0;
  const size_t raw = (size_t)B * (size_t)H * (size_t)Nq * sizeof(float);
  return (raw + 255) & ~size_t(255);
}

// gfx950 check, cached per device ordinal.
int check_device() {
  static std::mutex mu;
  static signed char arch_ok[64];  // 0 unknown, 1 ok, -1 unsupported
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (dev >= 64) return ATTN_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return arch_ok[dev] == 1 ? ATTN_OK : ATTN_ERR_DEVICE;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU holds its own copy at its own
// address); null if the lookup fails.
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

attn::MaskGeom make_geom(int mask, int64_t Nq, int64_t Nk, int64_t window) {
  attn::MaskGeom g;
  g.mode = mask;
  g.nq = (int)Nq;
  g.nk = (int)Nk;
  g.window = (mask == ATTN_MASK_SLIDING || mask == ATTN_MASK_BLOCK) ? (int)window : 0;
  g.window_q = mask == ATTN_MASK_BLOCK ? (int)(Nq / (Nk / window)) : 0;
  return g;
}

// The dK/dV pass keeps dS for the dQ pass (bf16, general kernels, d = 128):
// B * H * ds_blocks() blocks of 32 x 32 bf16 after the row sums.
bool ds_applies(int dtype, int64_t d, const attn::MaskGeom& g) {
  return is16(dtype) && d == 128 && !g.local64();
}

size_t ds_ws_size(int64_t B, int64_t H, int64_t Nq, const attn::MaskGeom& g) {
  return ws_size(B, H, Nq) + (size_t)B * (size_t)H * (size_t)g.ds_blocks() *
                                 (size_t)attn::kDsBlockElems * sizeof(uint16_t);
}

// bytes of the workspace a backward call uses: with room for the dS blocks
// (where they apply) the dS path, else the row sums only
size_t ws_used(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int mask,
               int64_t window, size_t workspace_bytes) {
  const attn::MaskGeom g = make_geom(mask, Nq, Nk, window);
  if (ds_applies(dtype, d, g)) {
    const size_t full = ds_ws_size(B, H, Nq, g);
    if (workspace_bytes >= full) return full;
  }
  return ws_size(B, H, Nq);
}

// ------------------------------------------------------- tensor arguments

constexpr int64_t kMaxStride = int64_t(1) << 48;      // elements
constexpr int64_t kMaxSliceSpan = int64_t(1) << 31;   // elements, row offsets in 31 bits

// One pointer argument: a [B][H][n][d] tensor at `lay` with window length T
// (tokens per window), or, when flat > 0, a contiguous buffer of `flat` bytes
// (lse, the workspace).
struct Arg {
  const void* p;
  attn_layout lay;
  int64_t n, T;
  size_t flat;
};

struct Dim {
  int64_t stride, extent;  // bytes, extent > 1
};

int64_t mul_sat(int64_t a, int64_t b) {  // a, b >= 0
  if (a != 0 && b > INT64_MAX / a) return INT64_MAX;
  return a * b;
}

int64_t add_sat(int64_t a, int64_t b) {  // a, b >= 0
  return a > INT64_MAX - b ? INT64_MAX : a + b;
}

struct Shape {
  int64_t B, H, d;
  size_t es;
};

// dimensions of extent > 1 of a tensor argument, in bytes, by stride
int dims_of(const Arg& t, const Shape& sh, Dim* dims) {
  const Dim all[4] = {{t.lay.batch, sh.B}, {t.lay.head, sh.H}, {t.lay.window, t.n / t.T},
                      {t.lay.token, t.T}};
  int nd = 0;
  for (const Dim& x : all)
    if (x.extent > 1) dims[nd++] = {mul_sat(x.stride, (int64_t)sh.es), x.extent};
  std::sort(dims, dims + nd, [](const Dim& x, const Dim& y) { return x.stride < y.stride; });
  return nd;
}

// strides in range, rows nested (no two rows of the tensor overlap), the
// rows of a slice within 2^31 elements of its first
bool layout_valid(const Arg& t, const Shape& sh) {
  const attn_layout& l = t.lay;
  for (int64_t st : {l.batch, l.head, l.window, l.token})
    if (st < 0 || st > kMaxStride) return false;
  Dim dims[4];
  const int nd = dims_of(t, sh, dims);
  int64_t need = sh.d * (int64_t)sh.es;
  for (int i = 0; i < nd; ++i) {
    if (dims[i].stride < need) return false;
    need = mul_sat(dims[i].stride, dims[i].extent);
  }
  const int64_t nwin = t.n / t.T;
  int64_t last = sh.d;
  if (nwin > 1) last = add_sat(last, mul_sat(nwin - 1, l.window));
  if (t.T > 1) last = add_sat(last, mul_sat(t.T - 1, l.token));
  return last <= kMaxSliceSpan;
}

bool strides_aligned(const Arg& t, const Shape& sh) {
  Dim dims[4];
  const int nd = dims_of(t, sh, dims);
  for (int i = 0; i < nd; ++i)
    if (dims[i].stride % 16) return false;
  return true;
}

// bytes from the base pointer to the end of the tensor's last element
int64_t span_bytes(const Arg& t, const Shape& sh) {
  if (t.flat) return (int64_t)t.flat;
  Dim dims[4];
  const int nd = dims_of(t, sh, dims);
  int64_t end = sh.d * (int64_t)sh.es;
  for (int i = 0; i < nd; ++i) end = add_sat(end, mul_sat(dims[i].stride, dims[i].extent - 1));
  return end;
}

// Is there a digit vector c (|c_k| < extent_k) with sum c_k stride_k within
// one row (|rest| < row bytes) of delta?  For nested dimensions the inner
// sum is smaller than the next stride, so at each level only the two nearest
// multiples of the stride can be part of a solution.
bool reaches(int64_t delta, const Dim* dims, int k, int64_t row) {
  if (k < 0) return delta > -row && delta < row;
  const int64_t s = dims[k].stride, n = dims[k].extent;
  int64_t q = delta / s;
  if (delta % s != 0 && delta < 0) --q;  // floor
  for (int64_t c = q; c <= q + 1; ++c)
    if (c > -n && c < n && reaches(delta - c * s, dims, k - 1, row)) return true;
  return false;
}

// Do two arguments share a byte?  Exact for two tensors with the same
// dimensions (interleaved views of one buffer), by address range otherwise.
bool args_overlap(const Arg& x, const Arg& y, const Shape& sh) {
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(x.p), y0 = reinterpret_cast<uintptr_t>(y.p);
  const int64_t xs = span_bytes(x, sh), ys = span_bytes(y, sh);
  if (!(x0 < y0 + (uint64_t)ys && y0 < x0 + (uint64_t)xs)) return false;
  if (x.flat || y.flat) return true;
  Dim dx[4], dy[4];
  const int nx = dims_of(x, sh, dx), ny = dims_of(y, sh, dy);
  if (nx != ny) return true;
  for (int i = 0; i < nx; ++i)
    if (dx[i].stride != dy[i].stride || dx[i].extent != dy[i].extent) return true;
  const int64_t delta = (int64_t)(y0 - x0);
  return reaches(delta, dx, nx - 1, sh.d * (int64_t)sh.es);
}

// The kernels' row map of a tensor argument, or false when its windows are
// interleaved with a window length that is not a power of two.
bool make_rowmap(const Arg& t, attn::RowMap* rm) {
  rm->batch = t.lay.batch;
  rm->head = t.lay.head;
  const int64_t nwin = t.n / t.T;
  if (nwin == 1 || t.lay.window == t.T * t.lay.token) {
    // one run of rows at the token stride
    rm->wshift = 31;
    rm->wmask = 0x7fffffff;
    rm->win = 0;
    rm->tok = (t.n > 1) ? (int32_t)(nwin > 1 && t.T == 1 ? t.lay.window : t.lay.token) : 0;
    return true;
  }
  if (t.T & (t.T - 1)) return false;
  int sh = 0;
  while ((int64_t(1) << sh) < t.T) ++sh;
  rm->wshift = sh;
  rm->wmask = (int32_t)(t.T - 1);
  rm->win = (int32_t)t.lay.window;
  rm->tok = t.T > 1 ? (int32_t)t.lay.token : 0;
  return true;
}

attn_layout contiguous_layout(int64_t H, int64_t n, int64_t T, int64_t d) {
  return attn_layout{H * n * d, n * d, T * d, d};
}

void fill_contiguous(int64_t H, int64_t Nq, int64_t Nk, int64_t d, const attn::MaskGeom& g,
                     attn_layouts* out) {
  const int64_t tq = g.mode == attn::kBlock ? g.window_q : Nq;
  const int64_t tk = g.mode == attn::kBlock ? g.window : Nk;
  const attn_layout lq = contiguous_layout(H, Nq, tq, d), lk = contiguous_layout(H, Nk, tk, d);
  *out = attn_layouts{lq, lk, lk, lq, lq, lq, lk, lk};
}

// Validation of the pointer arguments: `ins` may overlap each other, `outs`
// may overlap nothing.  Order of checks: null pointers, layouts
// (INVALID_ARG), base pointers and strides (MISALIGNED), row maps
// (UNSUPPORTED), overlaps (ALIAS).
int check_args(const Arg* ins, int nin, const Arg* outs, int nout, const Shape& sh) {
  for (int i = 0; i < nin; ++i)
    if (!ins[i].p) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < nout; ++i)
    if (!outs[i].p) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < nin + nout; ++i) {
    const Arg& t = i < nin ? ins[i] : outs[i - nin];
    if (!t.flat && !layout_valid(t, sh)) return ATTN_ERR_INVALID_ARG;
  }
  for (int i = 0; i < nin + nout; ++i) {
    const Arg& t = i < nin ? ins[i] : outs[i - nin];
    if (!aligned16(t.p) || (!t.flat && !strides_aligned(t, sh))) return ATTN_ERR_MISALIGNED;
  }
  for (int i = 0; i < nin + nout; ++i) {
    const Arg& t = i < nin ? ins[i] : outs[i - nin];
    attn::RowMap rm;
    if (!t.flat && !make_rowmap(t, &rm)) return ATTN_ERR_UNSUPPORTED;
  }
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (args_overlap(outs[o], ins[i], sh)) return ATTN_ERR_ALIAS;
    for (int p = o + 1; p < nout; ++p)
      if (args_overlap(outs[o], outs[p], sh)) return ATTN_ERR_ALIAS;
  }
  return ATTN_OK;
}

Arg tensor_arg(const void* p, const attn_layout& lay, int64_t n, int64_t T) {
  return Arg{p, lay, n, T, 0};
}

Arg flat_arg(const void* p, size_t bytes) { return Arg{p, attn_layout{0, 0, 0, 0}, 1, 1, bytes}; }

// window lengths of query-side and key-side tensors
int64_t t_q(const attn::MaskGeom& g, int64_t Nq) { return g.mode == attn::kBlock ? g.window_q : Nq; }
int64_t t_k(const attn::MaskGeom& g, int64_t Nk) { return g.mode == attn::kBlock ? g.window : Nk; }

int check_fwd_impl(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                   int mask, int64_t window, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const attn_layouts* layouts) {
  int st = check_geometry(dtype, B, H, Nq, Nk, d, scale, mask, window);
  if (st) return st;
  const attn::MaskGeom g = make_geom(mask, Nq, Nk, window);
  attn_layouts cont;
  if (!layouts) {
    fill_contiguous(H, Nq, Nk, d, g, &cont);
    layouts = &cont;
  }
  const Shape sh{B, H, d, elem_size(dtype)};
  const int64_t tq = t_q(g, Nq), tk = t_k(g, Nk);
  const Arg ins[3] = {tensor_arg(q, layouts->q, Nq, tq), tensor_arg(k, layouts->k, Nk, tk),
                      tensor_arg(v, layouts->v, Nk, tk)};
  const Arg outs[2] = {tensor_arg(o, layouts->o, Nq, tq),
                       flat_arg(lse, (size_t)(B * H * Nq) * sizeof(float))};
  return check_args(ins, 3, outs, 2, sh);
}

int check_bwd_impl(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                   int mask, int64_t window, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const void* dout, const void* dq,
                   const void* dk, const void* dv, const void* workspace, size_t workspace_bytes,
                   const attn_layouts* layouts) {
  int st = check_geometry(dtype, B, H, Nq, Nk, d, scale, mask, window);
  if (st) return st;
  const attn::MaskGeom g = make_geom(mask, Nq, Nk, window);
  attn_layouts cont;
  if (!layouts) {
    fill_contiguous(H, Nq, Nk, d, g, &cont);
    layouts = &cont;
  }
  const Shape sh{B, H, d, elem_size(dtype)};
  const int64_t tq = t_q(g, Nq), tk = t_k(g, Nk);
  const Arg ins[6] = {tensor_arg(q, layouts->q, Nq, tq),       tensor_arg(k, layouts->k, Nk, tk),
                      tensor_arg(v, layouts->v, Nk, tk),       tensor_arg(o, layouts->o, Nq, tq),
                      flat_arg(lse, (size_t)(B * H * Nq) * sizeof(float)),
                      tensor_arg(dout, layouts->dout, Nq, tq)};
  if (!workspace) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < ws_size(B, H, Nq)) return ATTN_ERR_WORKSPACE;
  const Arg outs[4] = {tensor_arg(dq, layouts->dq, Nq, tq), tensor_arg(dk, layouts->dk, Nk, tk),
                       tensor_arg(dv, layouts->dv, Nk, tk),
                       flat_arg(workspace, ws_used(dtype, B, H, Nq, Nk, d, mask, window,
                                                   workspace_bytes))};
  return check_args(ins, 6, outs, 4, sh);
}

// row maps of validated arguments
attn::RowMap rowmap(const attn_layout& lay, int64_t n, int64_t T) {
  attn::RowMap rm;
  make_rowmap(tensor_arg(nullptr, lay, n, T), &rm);
  return rm;
}

// ------------------------------------------------------------ IHA premix

constexpr int64_t kPremixMaxH = 32;    // source heads (one MFMA column)
constexpr int64_t kPremixMaxHP = 128;  // pseudo-heads H * P (four MFMA tiles)
constexpr int64_t kPremixGrid = 1024;  // workgroups, and dW partials, per call

int premix_grid(int64_t B, int64_t N) { return (int)std::min<int64_t>(B * N, kPremixGrid); }

int check_premix_geometry(int dtype, int64_t B, int64_t N, int64_t H, int64_t P, int64_t d) {
  if (!is16(dtype)) return ATTN_ERR_UNSUPPORTED;
  if (B < 1 || N < 1 || H < 1 || P < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (!supported_d(d)) return ATTN_ERR_UNSUPPORTED;
  if (H > kPremixMaxH || H * P > kPremixMaxHP || (P & (P - 1))) return ATTN_ERR_UNSUPPORTED;
  if (N > kMaxSeq || B * N > (int64_t(1) << 40)) return ATTN_ERR_INVALID_ARG;
  // row offsets of one batch's output in 31 bits
  if (H * N * P * d >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

attn::PremixArgs premix_args(int64_t B, int64_t N, int64_t H, int64_t P) {
  attn::PremixArgs a{};
  a.B = (int)B;
  a.N = (int)N;
  a.H = (int)H;
  int lp = 0;
  while ((int64_t(1) << lp) < P) ++lp;
  a.lp = lp;
  a.grid = premix_grid(B, N);
  return a;
}

}  // namespace

extern "C" {

int attn_check_fwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   float scale, int mask, int64_t window, const void* q, const void* k,
                   const void* v, const void* o, const float* lse) {
  return check_fwd_impl(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse, nullptr);
}

int attn_check_bwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   float scale, int mask, int64_t window, const void* q, const void* k,
                   const void* v, const void* o, const float* lse, const void* dout,
                   const void* dq, const void* dk, const void* dv, const void* workspace,
                   size_t workspace_bytes) {
  return check_bwd_impl(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse, dout, dq,
                        dk, dv, workspace, workspace_bytes, nullptr);
}

int attn_check_fwd_strided(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                           float scale, int mask, int64_t window, const void* q, const void* k,
                           const void* v, const void* o, const float* lse,
                           const attn_layouts* layouts) {
  return check_fwd_impl(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse, layouts);
}

int attn_check_bwd_strided(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                           float scale, int mask, int64_t window, const void* q, const void* k,
                           const void* v, const void* o, const float* lse, const void* dout,
                           const void* dq, const void* dk, const void* dv, const void* workspace,
                           size_t workspace_bytes, const attn_layouts* layouts) {
  return check_bwd_impl(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse, dout, dq,
                        dk, dv, workspace, workspace_bytes, layouts);
}

int attn_layouts_contiguous(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int mask,
                            int64_t window, attn_layouts* out) {
  if (!out) return ATTN_ERR_INVALID_ARG;
  const int st = check_geometry(ATTN_BF16, B, H, Nq, Nk, d, 1.0f, mask, window);
  if (st) return ATTN_ERR_INVALID_ARG;
  fill_contiguous(H, Nq, Nk, d, make_geom(mask, Nq, Nk, window), out);
  return ATTN_OK;
}

size_t attn_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq) { return ws_size(B, H, Nq); }

size_t attn_bwd_workspace_size_ds(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                  int64_t d, int mask, int64_t window) {
  if (check_geometry(dtype, B, H, Nq, Nk, d, 1.0f, mask, window) != ATTN_OK) return 0;
  const attn::MaskGeom g = make_geom(mask, Nq, Nk, window);
  return ds_applies(dtype, d, g) ? ds_ws_size(B, H, Nq, g) : ws_size(B, H, Nq);
}

int attn_bwd_fused(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int mask,
                   int64_t window) {
  if (check_geometry(dtype, B, H, Nq, Nk, d, 1.0f, mask, window) != ATTN_OK) return 0;
  if (!is16(dtype)) return 0;
  const attn::MaskGeom g = make_geom(mask, Nq, Nk, window);
  if (g.local64()) return 1;
  return attn::short_keys(g, (int)d) ? 2 : 0;
}

int attn_fwd_strided(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                     float scale, int mask, int64_t window, const void* q, const void* k,
                     const void* v, void* o, float* lse, const attn_layouts* layouts,
                     void* stream) {
  int st = check_fwd_impl(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse, layouts);
  if (st) return st;
  st = check_device();
  if (st) return st;
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = (int)B;
  a.H = (int)H;
  a.nq = (int)Nq;
  a.nk = (int)Nk;
  a.scale = scale;
  a.mg = make_geom(mask, Nq, Nk, window);
  attn_layouts cont;
  if (!layouts) {
    fill_contiguous(H, Nq, Nk, d, a.mg, &cont);
    layouts = &cont;
  }
  const int64_t tq = t_q(a.mg, Nq), tk = t_k(a.mg, Nk);
  a.rq = rowmap(layouts->q, Nq, tq);
  a.rk = rowmap(layouts->k, Nk, tk);
  a.rv = rowmap(layouts->v, Nk, tk);
  a.ro = rowmap(layouts->o, Nq, tq);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int err = is16(dtype) ? attn::launch_fwd_16(a, dtype == ATTN_FP16, (int)d, s)
                              : attn::launch_fwd_fp32(a, (int)d, s);
  return err ? ATTN_ERR_LAUNCH : ATTN_OK;
}

int attn_fwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
             int mask, int64_t window, const void* q, const void* k, const void* v, void* o,
             float* lse, void* stream) {
  return attn_fwd_strided(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse, nullptr,
                          stream);
}

int attn_bwd_strided(int passes, int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                     int64_t d, float scale, int mask, int64_t window, const void* q,
                     const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, const attn_layouts* layouts, void* stream) {
  if (passes < 1 || passes > ATTN_PASS_ALL) return ATTN_ERR_INVALID_ARG;
  if (passes != ATTN_PASS_ALL && attn_bwd_fused(dtype, B, H, Nq, Nk, d, mask, window) == 1)
    return ATTN_ERR_UNSUPPORTED;
  int st = check_bwd_impl(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse, dout, dq,
                          dk, dv, workspace, workspace_bytes, layouts);
  if (st) return st;
  st = check_device();
  if (st) return st;
  attn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsum = static_cast<float*>(workspace);
  a.B = (int)B;
  a.H = (int)H;
  a.nq = (int)Nq;
  a.nk = (int)Nk;
  a.scale = scale;
  a.mg = make_geom(mask, Nq, Nk, window);
  a.ds = nullptr;
  a.ds_per_bh = 0;
  if (ws_used(dtype, B, H, Nq, Nk, d, mask, window, workspace_bytes) > ws_size(B, H, Nq)) {
    a.ds = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + ws_size(B, H, Nq));
    a.ds_per_bh = a.mg.ds_blocks();
  }
  attn_layouts cont;
  if (!layouts) {
    fill_contiguous(H, Nq, Nk, d, a.mg, &cont);
    layouts = &cont;
  }
  const int64_t tq = t_q(a.mg, Nq), tk = t_k(a.mg, Nk);
  a.rq = rowmap(layouts->q, Nq, tq);
  a.rk = rowmap(layouts->k, Nk, tk);
  a.rv = rowmap(layouts->v, Nk, tk);
  a.ro = rowmap(layouts->o, Nq, tq);
  a.rdo = rowmap(layouts->dout, Nq, tq);
  a.rdq = rowmap(layouts->dq, Nq, tq);
  a.rdk = rowmap(layouts->dk, Nk, tk);
  a.rdv = rowmap(layouts->dv, Nk, tk);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int err = is16(dtype) ? attn::launch_bwd_16(a, dtype == ATTN_FP16, (int)d, s, passes)
                              : attn::launch_bwd_fp32(a, (int)d, s, passes);
  return err ? ATTN_ERR_LAUNCH : ATTN_OK;
}

int attn_bwd_passes(int passes, int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                    int64_t d, float scale, int mask, int64_t window, const void* q,
                    const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return attn_bwd_strided(passes, dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse,
                          dout, dq, dk, dv, workspace, workspace_bytes, nullptr, stream);
}

int attn_bwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
             int mask, int64_t window, const void* q, const void* k, const void* v,
             const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_passes(ATTN_PASS_ALL, dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o,
                         lse, dout, dq, dk, dv, workspace, workspace_bytes, stream);
}

int attn_bwd_noalloc(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                     float scale, int mask, int64_t window, const void* q, const void* k,
                     const void* v, const void* o, const float* lse, const void* dout, void* dq,
                     void* dk, void* dv, void* stream) {
  int st = check_geometry(dtype, B, H, Nq, Nk, d, scale, mask, window);
  if (st) return st;
  // the minimum workspace: row sums only, so the dQ pass recomputes
  const size_t need = ws_size(B, H, Nq);
  if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
  st = check_device();
  if (st) return st;
  void* ws = scratch_ptr();
  if (!ws) return ATTN_ERR_DEVICE;
  return attn_bwd(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse, dout, dq, dk, dv,
                  ws, need, stream);
}

// ------------------------------------------------------------ IHA premix

size_t attn_premix_bwd_workspace_size(int64_t B, int64_t N, int64_t H, int64_t P) {
  if (B < 1 || N < 1 || H < 1 || P < 1 || H > kPremixMaxH || H * P > kPremixMaxHP) return 0;
  const size_t raw = (size_t)premix_grid(B, N) * (size_t)(H * P * H) * sizeof(float);
  return (raw + 255) & ~size_t(255);
}

int attn_check_premix_fwd(int dtype, int64_t B, int64_t N, int64_t H, int64_t P, int64_t d,
                          const void* x, const void* w, const void* out) {
  int st = check_premix_geometry(dtype, B, N, H, P, d);
  if (st) return st;
  const size_t es = elem_size(dtype);
  const Arg ins[2] = {flat_arg(x, (size_t)(B * N * H * d) * es), flat_arg(w, (size_t)(H * P * H) * es)};
  const Arg outs[1] = {flat_arg(out, (size_t)(B * H * N * P * d) * es)};
  return check_args(ins, 2, outs, 1, Shape{B, H, d, es});
}

int attn_check_premix_bwd(int dtype, int64_t B, int64_t N, int64_t H, int64_t P, int64_t d,
                          const void* x, const void* w, const void* dout, const void* dx,
                          const float* dw, const void* workspace, size_t workspace_bytes) {
  int st = check_premix_geometry(dtype, B, N, H, P, d);
  if (st) return st;
  const size_t es = elem_size(dtype);
  const Arg ins[3] = {flat_arg(x, (size_t)(B * N * H * d) * es),
                      flat_arg(w, (size_t)(H * P * H) * es),
                      flat_arg(dout, (size_t)(B * H * N * P * d) * es)};
  if (!workspace || workspace_bytes < attn_premix_bwd_workspace_size(B, N, H, P))
    return ATTN_ERR_WORKSPACE;
  const Arg outs[3] = {flat_arg(dx, (size_t)(B * N * H * d) * es),
                       flat_arg(dw, (size_t)(H * P * H) * sizeof(float)),
                       flat_arg(workspace, attn_premix_bwd_workspace_size(B, N, H, P))};
  return check_args(ins, 3, outs, 3, Shape{B, H, d, es});
}

int attn_premix_fwd(int dtype, int64_t B, int64_t N, int64_t H, int64_t P, int64_t d,
                    const void* x, const void* w, void* out, void* stream) {
  int st = attn_check_premix_fwd(dtype, B, N, H, P, d, x, w, out);
  if (st) return st;
  st = check_device();
  if (st) return st;
  attn::PremixArgs a = premix_args(B, N, H, P);
  a.x = x;
  a.w = w;
  a.out = out;
  const int err = attn::launch_premix_fwd(a, dtype == ATTN_FP16, (int)d,
                                          static_cast<hipStream_t>(stream));
  return err ? ATTN_ERR_LAUNCH : ATTN_OK;
}

int attn_premix_bwd(int dtype, int64_t B, int64_t N, int64_t H, int64_t P, int64_t d,
                    const void* x, const void* w, const void* dout, void* dx, float* dw,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = attn_check_premix_bwd(dtype, B, N, H, P, d, x, w, dout, dx, dw, workspace,
                                 workspace_bytes);
  if (st) return st;
  st = check_device();
  if (st) return st;
  attn::PremixArgs a = premix_args(B, N, H, P);
  a.x = x;
  a.w = w;
  a.dout = dout;
  a.dx = dx;
  a.dw = dw;
  a.dw_part = static_cast<float*>(workspace);
  const int err = attn::launch_premix_bwd(a, dtype == ATTN_FP16, (int)d,
                                          static_cast<hipStream_t>(stream));
  return err ? ATTN_ERR_LAUNCH : ATTN_OK;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_MISALIGNED: return "ATTN_ERR_MISALIGNED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_ALIAS: return "ATTN_ERR_ALIAS";
    case ATTN_ERR_DEVICE: return "ATTN_ERR_DEVICE";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH";
  }
  return "ATTN_ERR_UNKNOWN";
}

}  // extern "C"
