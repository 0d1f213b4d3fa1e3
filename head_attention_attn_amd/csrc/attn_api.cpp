// attn_api.cpp -- the C ABI of include/attn.h: argument validation, device
// gating and dispatch to the kernel launchers.  No device memory is allocated
// here and no state is kept per call; the only global state is a per-device
// cache of "is this a gfx950", filled once under a mutex.
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

namespace {

constexpr int64_t kMaxSeq = int64_t(1) << 30;   // per-(b,h) row counts fit int32 math
constexpr int64_t kMaxGrid = INT_MAX;           // 1-D grid of workgroups

bool supported_d(int64_t d) { return d == 64 || d == 96 || d == 128; }

size_t elem_size(int dtype) { return dtype == ATTN_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const void* p;
  size_t bytes;
};

bool overlap(Span a, Span b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Common checks of sizes, dtype, d, mask and window.
int check_geometry(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   float scale, int mask, int64_t window) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return ATTN_ERR_UNSUPPORTED;
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

int check_buffers(const Span* ins, int nin, const Span* outs, int nout) {
  for (int i = 0; i < nin; ++i)
    if (!ins[i].p) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < nout; ++i)
    if (!outs[i].p) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < nin; ++i)
    if (!aligned16(ins[i].p)) return ATTN_ERR_MISALIGNED;
  for (int i = 0; i < nout; ++i)
    if (!aligned16(outs[i].p)) return ATTN_ERR_MISALIGNED;
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlap(outs[o], ins[i])) return ATTN_ERR_ALIAS;
    for (int p = o + 1; p < nout; ++p)
      if (overlap(outs[o], outs[p])) return ATTN_ERR_ALIAS;
  }
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
  static signed char verdict[64];  // 0 unknown, 1 ok, -1 unsupported
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (dev >= 64) return ATTN_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (verdict[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    verdict[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return verdict[dev] == 1 ? ATTN_OK : ATTN_ERR_DEVICE;
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
  return dtype == ATTN_BF16 && d == 128 && !g.local64();
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

}  // namespace

extern "C" {

int attn_check_fwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   float scale, int mask, int64_t window, const void* q, const void* k,
                   const void* v, const void* o, const float* lse) {
  int st = check_geometry(dtype, B, H, Nq, Nk, d, scale, mask, window);
  if (st) return st;
  const size_t es = elem_size(dtype);
  const size_t qb = (size_t)(B * H * Nq * d) * es, kb = (size_t)(B * H * Nk * d) * es;
  const Span ins[3] = {{q, qb}, {k, kb}, {v, kb}};
  const Span outs[2] = {{o, qb}, {lse, (size_t)(B * H * Nq) * sizeof(float)}};
  return check_buffers(ins, 3, outs, 2);
}

int attn_check_bwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   float scale, int mask, int64_t window, const void* q, const void* k,
                   const void* v, const void* o, const float* lse, const void* dout,
                   const void* dq, const void* dk, const void* dv, const void* workspace,
                   size_t workspace_bytes) {
  int st = check_geometry(dtype, B, H, Nq, Nk, d, scale, mask, window);
  if (st) return st;
  const size_t es = elem_size(dtype);
  const size_t qb = (size_t)(B * H * Nq * d) * es, kb = (size_t)(B * H * Nk * d) * es;
  const size_t lb = (size_t)(B * H * Nq) * sizeof(float);
  const Span ins[6] = {{q, qb}, {k, kb}, {v, kb}, {o, qb}, {lse, lb}, {dout, qb}};
  if (!workspace) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < ws_size(B, H, Nq)) return ATTN_ERR_WORKSPACE;
  const Span outs[4] = {{dq, qb}, {dk, kb}, {dv, kb},
                        {workspace, ws_used(dtype, B, H, Nq, Nk, d, mask, window, workspace_bytes)}};
  return check_buffers(ins, 6, outs, 4);
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
  if (dtype != ATTN_BF16) return 0;
  return make_geom(mask, Nq, Nk, window).local64() ? 1 : 0;
}

int attn_fwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
             int mask, int64_t window, const void* q, const void* k, const void* v, void* o,
             float* lse, void* stream) {
  int st = attn_check_fwd(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse);
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int err = dtype == ATTN_BF16 ? attn::launch_fwd_bf16(a, (int)d, s)
                                     : attn::launch_fwd_fp32(a, (int)d, s);
  return err ? ATTN_ERR_LAUNCH : ATTN_OK;
}

int attn_bwd_passes(int passes, int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                    int64_t d, float scale, int mask, int64_t window, const void* q,
                    const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (passes < 1 || passes > ATTN_PASS_ALL) return ATTN_ERR_INVALID_ARG;
  if (passes != ATTN_PASS_ALL && attn_bwd_fused(dtype, B, H, Nq, Nk, d, mask, window) == 1)
    return ATTN_ERR_UNSUPPORTED;
  int st = attn_check_bwd(dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o, lse, dout,
                          dq, dk, dv, workspace, workspace_bytes);
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int err = dtype == ATTN_BF16 ? attn::launch_bwd_bf16(a, (int)d, s, passes)
                                     : attn::launch_bwd_fp32(a, (int)d, s, passes);
  return err ? ATTN_ERR_LAUNCH : ATTN_OK;
}

int attn_bwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
             int mask, int64_t window, const void* q, const void* k, const void* v,
             const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_passes(ATTN_PASS_ALL, dtype, B, H, Nq, Nk, d, scale, mask, window, q, k, v, o,
                         lse, dout, dq, dk, dv, workspace, workspace_bytes, stream);
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
