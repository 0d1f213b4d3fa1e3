"""Throughput of fused attention forward + backward on one MI355X.

One step = the whole hot path over one batch of synthetic input already
resident in HBM: ``attn_fwd`` (O and lse), then the backward -- the three
passes (row sums D, dK/dV, dQ) through ``attn_bwd_passes``, or the one fused
kernel where the library fuses them -- all on torch's current stream.  W
untimed warmup steps, then K timed steps bracketed by a device
synchronisation on both sides.  HIP events recorded between the calls, on the
stream the kernels run on, give each kernel's average duration over the timed
region.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value      algorithmic TFLOP/s of the headline workload's step: (4 d + 10 d)
             flops per visible (query, key) pair (forward 4 d, backward 10 d)
             over the step time
  roofline   the kernel with the largest share of the step: its algorithmic
             flops (MFMA-bound workloads) or compulsory bytes (HBM-bound ones)
             per launch over its measured average duration, against the
             MI355X peak.  The bound is the step's: its flops over the bytes
             the method must move (read Q, K, V, write O, lse; read Q, K, V,
             O, dO, lse, write dQ, dK, dV) against the ridge point.
             ``traffic`` is the HBM bytes per launch that rocprofv3 counters
             measured for that kernel (profiles/traffic_<workload>.txt), or
             null when the kernel sources changed since
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
             workload on this host, in the same unit
  parity     GPU outputs of the sampled slices against the oracle, checked
             outside the timed region
  timing     p10 / median / p90 of the step and of each kernel over the timed
             steps ("warm": back to back) and over steps each preceded by a
             1 GiB read that evicts every cache ("cache_flushed"), with the
             dominant kernel's roofline fraction at each median
  configs    one entry per benchmark configuration (the exact fp32 check, the
             Hiera mask-unit windows, the Hiera global stage, the causal LM and
             the causal sliding window over pseudo-heads): step time spread,
             TFLOP/s, per-kernel medians, the dominant kernel's roofline
             fraction under the step's bound, its counter traffic, and
             sampled-slice parity against the oracle

Workloads (``--workload``): causal_lm (default; 20 heads, N = 8192, d = 128,
causal), sliding_pseudo_head, block_local_hiera, block_pooled_hiera,
global_vision, iha_joint, tiny_exact_fp32.  ``--gpus`` above 1 is refused:
this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 (and fp16) MFMA, AMD published
FP32_VECTOR_PEAK_TFLOPS = 157.3

KERNELS = ("fwd", "rowsum", "dkdv", "dq")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ work accounting

def row_intervals(mask: str, window: int, nq: int, nk: int):
    """Visible key interval [lo, hi) of every query row (closed forms)."""
    i = np.arange(nq, dtype=np.int64)
    if mask == "none":
        lo, hi = np.zeros_like(i), np.full_like(i, nk)
    elif mask == "causal":
        lo, hi = np.zeros_like(i), np.minimum(i + 1, nk)
    elif mask == "sliding":
        lo, hi = np.maximum(0, i - window + 1), np.minimum(i + 1, nk)
    elif mask == "block":
        # nk / window windows of `window` keys, nq / (nk / window) query rows each
        wq = nq // (nk // window)
        lo = (i // wq) * window
        hi = np.minimum(lo + window, nk)
    else:
        raise ValueError(mask)
    return lo, np.maximum(hi, lo)


def visible_pairs(mask: str, window: int, nq: int, nk: int) -> int:
    """Number of visible (query, key) pairs of one (batch, head)."""
    lo, hi = row_intervals(mask, window, nq, nk)
    return int((hi - lo).sum())


def kernel_work(w, pairs_per_bh: int, kept_ds: bool = False) -> dict:
    """Algorithmic flops and compulsory HBM bytes per launch of each kernel.

    flops per visible pair: fwd 4 d (Q K^T and P V); dK/dV pass 8 d (S, dP,
    dV, dK); dQ pass 2 d (the dQ product; when it recomputes S and dP those
    are not credited), so the backward totals 10 d, which is also what the
    fused backward is credited with.  ``bytes``: every tensor the method's
    step must read or write, once.  With ``kept_ds`` the dK/dV pass also
    writes dS (bf16, 2 bytes per visible pair) and the dQ pass reads it back
    instead of recomputing it: that workspace is this library's choice, not
    the method's traffic, so it is reported apart as ``workspace_bytes`` and
    never decides a bound."""
    es = 4 if w.dtype == "fp32" else 2
    bh = w.B * w.H
    q_rows, k_rows, d = bh * w.Nq, bh * w.Nk, w.d
    pairs = bh * pairs_per_bh
    ds_bytes = 2 * pairs if kept_ds else 0
    return {
        "fwd": dict(flops=4 * d * pairs, workspace_bytes=0,
                    bytes=(2 * q_rows * d + 2 * k_rows * d) * es + 4 * q_rows),
        "rowsum": dict(flops=2 * d * q_rows, bytes=2 * q_rows * d * es + 4 * q_rows,
                       workspace_bytes=0),
        "dkdv": dict(flops=8 * d * pairs, workspace_bytes=ds_bytes,
                     bytes=(2 * q_rows * d + 4 * k_rows * d) * es + 8 * q_rows),
        "dq": dict(flops=2 * d * pairs, workspace_bytes=ds_bytes,
                   bytes=(3 * q_rows * d + 2 * k_rows * d) * es + 8 * q_rows),
        # the fused backward: reads Q, K, V, dO, lse, writes dQ, dK, dV (its
        # row sums come from P and dP in-tile, O is not read)
        "bwd": dict(flops=10 * d * pairs, workspace_bytes=0,
                    bytes=(3 * q_rows * d + 4 * k_rows * d) * es + 4 * q_rows),
    } | premix_work(w, es)


def step_work(w, pairs_per_bh: int) -> dict:
    """The step's algorithmic flops (14 d per visible pair), the bytes the
    method must move (forward: read Q, K, V, write O, lse; backward: read Q,
    K, V, O, dO, lse, write dQ, dK, dV), and what bounds it: MFMA (or the
    fp32 vector ALUs) above the ridge point, HBM below it, launch latency
    when either roofline time is under 2 us (the exact-check config)."""
    es = 4 if w.dtype == "fp32" else 2
    bh = w.B * w.H
    q_rows, k_rows, d = bh * w.Nq, bh * w.Nk, w.d
    flops = 14 * d * bh * pairs_per_bh
    nbytes = (6 * q_rows * d + 6 * k_rows * d) * es + 8 * q_rows
    peak = FP32_VECTOR_PEAK_TFLOPS if w.dtype == "fp32" else MFMA_BF16_PEAK_TFLOPS
    t_math = flops / (peak * 1e12)
    t_mem = nbytes / (HBM_PEAK_GBS * 1e9)
    if max(t_math, t_mem) < 2e-6:
        bound = "latency"
    elif t_math >= t_mem:
        bound = "alu" if w.dtype == "fp32" else "mfma"
    else:
        bound = "hbm"
    return {"flops": flops, "bytes": nbytes, "bound": bound, "peak": peak,
            "roofline_ms": max(t_math, t_mem) * 1e3,
            "arithmetic_intensity": round(flops / nbytes, 2)}


def kernel_roofline(wk: dict, bound: str, peak: float, ms: float):
    """A kernel's achieved rate under the step's bound and its fraction of
    the peak: flops over its duration for MFMA / ALU bounds, compulsory bytes
    over its duration for HBM; None for a latency-bound step."""
    t = ms * 1e-3
    if bound in ("mfma", "alu"):
        a = wk["flops"] / t / 1e12
        return {"bound": bound, "achieved": round(a, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(a / peak, 4)}
    if bound == "hbm":
        a = wk["bytes"] / t / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4)}
    return None


def premix_work(w, es: int) -> dict:
    """IHA premix of Q, K and V (three launches each way): per tensor the
    forward reads X [B][N][H][d] and W and writes the B*H*N*P*d pseudo-token
    elements (2 H flops each); the backward reads X and dOut, writes dX (2 H P
    flops per element) and dW (2 per pseudo-token element), plus the fp32 dW
    partials written and read once."""
    if w.P <= 1:
        return {}
    N = w.Nq // w.P
    x = w.B * N * w.H * w.d
    y = x * w.P
    wt = w.H * w.P * w.H
    part = min(w.B * N, 1024) * wt * 4
    return {
        "premix": dict(flops=3 * 2 * w.H * y, bytes=3 * ((x + y + wt) * es)),
        "premix_bwd": dict(flops=3 * (2 * w.H * w.P * x + 2 * y * w.H),
                           bytes=3 * ((2 * x + y + wt) * es + 2 * part + wt * 4)),
    }


def source_digest() -> str:
    """sha256 over the kernel sources, to tell whether stored counter
    readings still describe the kernels being timed."""
    csrc = os.path.join(ROOT, "head_attention_attn_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch from profiles/traffic_<workload>.txt when it was
    taken from the current kernel sources, else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != source_digest():
        return None
    val = fields.get(f"traffic_bytes_per_launch.{kernel}")
    return float(val) if val is not None else None


def step_spread(events, kernels) -> dict:
    """p10 / median / p90 of the step time and of each kernel's time over
    the steps, from HIP events recorded before the step and after each
    kernel of it."""
    def pct(xs):
        a = np.asarray(xs, dtype=np.float64)
        return {"p10": round(float(np.percentile(a, 10)), 5),
                "median": round(float(np.median(a)), 5),
                "p90": round(float(np.percentile(a, 90)), 5)}
    return {"ms_per_step": pct([e[0].elapsed_time(e[-1]) for e in events]),
            "per_kernel_ms": {kn: pct([e[i].elapsed_time(e[i + 1]) for e in events])
                              for i, kn in enumerate(kernels)}}


def stored_clock(workload: str, kernel: str):
    """The clock (GHz) the kernel ran at in the rocprofv3 counter run of
    profiles/mfma_<workload>.txt (GRBM_GUI_ACTIVE cycles over the dispatch
    duration), when that run was taken from the current kernel sources and
    the kernel was long enough to time it; else None."""
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}.txt")
    if not os.path.exists(path):
        return None
    digest, clock = None, None
    with open(path) as f:
        for line in f:
            if line.startswith("source_sha256:"):
                digest = line.split(":", 1)[1].strip()
            parts = line.split()
            if len(parts) >= 3 and parts[0] == kernel:
                try:
                    clock = float(parts[2])
                except ValueError:
                    clock = None
    return clock if digest == source_digest() else None


# ------------------------------------------------------- interleaved heads

def iha_setup(attn, torch, w, dev):
    """Inputs of the IHA premix for Q, K, V (seeds 100, 101, 102), their
    pseudo-token outputs and the backward's buffers."""
    from head_attention_attn_amd.inputs import make_premix_inputs
    N = w.Nq // w.P
    xs, ws = [], []
    for i in range(3):
        x, wt, _ = make_premix_inputs(w.B, N, w.H, w.P, w.d, w.dtype, seed=100 + i)
        xs.append(x.to(dev))
        ws.append(wt.to(dev))
    out = [attn.binding.premix(x, wt) for x, wt in zip(xs, ws)]
    torch.cuda.synchronize(dev)
    return {"x": xs, "w": ws, "out": out,
            "dx": [torch.empty_like(x) for x in xs],
            "dw": [torch.empty((w.H, w.P, w.H), dtype=torch.float32, device=dev) for _ in xs],
            "ws": torch.empty(attn.binding.premix_workspace_bytes(w.B, N, w.H, w.P),
                              dtype=torch.uint8, device=dev)}


def premix_parity(iha, w, npos: int = 32):
    """The first ``npos`` positions of the Q premix against the oracle:
    max |gpu - ref| / bound.  The fp32 sum s of H products is within
    H 2^-24 sum|terms| of ref, and rounding it to bf16 adds at most 2^-8 |s|
    <= 2^-8 (|ref| + |s - ref|), so the bound is
    2^-8 |ref| + (1 + 2^-8) H 2^-24 sum|terms|."""
    import numpy as np
    from oracle.premix import premix_fwd
    x = iha["x"][0][:, :npos].double().cpu().numpy()
    wt = iha["w"][0].double().cpu().numpy()
    ref = premix_fwd(x, wt)
    absref = premix_fwd(np.abs(x), np.abs(wt))
    got = iha["out"][0][:, :, :npos].double().cpu().numpy()
    u = 2.0 ** -8
    bound = u * np.abs(ref) + (1 + u) * w.H * 2.0 ** -24 * absref + 1e-30
    return float(np.max(np.abs(got - ref) / bound))


# ------------------------------------------------------- Hiera token order

def token_order_timing(attn, torch, w, q, k, v, do, ws, kw, fused, o_ref, lse_ref, dq_ref, dk_ref,
                       dv_ref, steps, dev):
    """The block-mask step with its tensors in Hiera's token order (token
    n = t * nw + w, window index fastest): K and V interleaved in one
    (B, T, nw, 3, H, d) projection buffer, Q and dO in (B, Tq, nw, H, d)
    buffers, O and dQ written in that order and dK, dV into one interleaved
    (B, T, nw, 2, H, d) buffer -- read and written in place through the
    strided entry points.  Against it, the same step on the contiguous
    window-major layout plus the copies into and out of it that a caller
    without strided kernels makes."""
    B, H, d = w.B, w.H, w.d
    nw = w.Nk // w.window
    T, Tq = w.window, w.Nq // nw
    qkv = torch.empty((B, T, nw, 3, H, d), dtype=q.dtype, device=dev)
    qbuf = torch.empty((B, Tq, nw, H, d), dtype=q.dtype, device=dev)
    gbuf = torch.empty_like(qbuf)
    obuf, dqbuf = torch.empty_like(qbuf), torch.empty_like(qbuf)
    dkv = torch.empty((B, T, nw, 2, H, d), dtype=q.dtype, device=dev)

    def split(buf, slot=None):            # [B, nw, H, T, d] view
        x = buf if slot is None else buf[:, :, :, slot]
        return x.permute(0, 2, 3, 1, 4)

    def windows(x4, t):                   # [B, H, nw*t, d] -> [B, nw, H, t, d] view
        return x4.view(B, H, nw, t, d).permute(0, 2, 1, 3, 4)

    q5, g5, o5, dq5 = split(qbuf), split(gbuf), split(obuf), split(dqbuf)
    k5, v5, dk5, dv5 = split(qkv, 1), split(qkv, 2), split(dkv, 0), split(dkv, 1)
    q5.copy_(windows(q, Tq))
    g5.copy_(windows(do, Tq))
    k5.copy_(windows(k, T))
    v5.copy_(windows(v, T))
    skw = dict(scale=w.scale)

    def strided_step():
        attn.fwd(q5, k5, v5, out=o5, lse=lse_t, **skw)
        attn.bwd(q5, k5, v5, o5, lse_t, g5, workspace=ws, dq=dq5, dk=dk5, dv=dv5, **skw)

    qc, kc, vc, gc = (torch.empty_like(t) for t in (q, k, v, do))
    oc, dqc, dkc, dvc = (torch.empty_like(t) for t in (q, q, k, v))
    lse_t = torch.empty_like(lse_ref)
    lse_c = torch.empty_like(lse_ref)

    def copy_step():
        for dst, src, t in ((qc, q5, Tq), (kc, k5, T), (vc, v5, T), (gc, g5, Tq)):
            windows(dst, t).copy_(src)
        attn.fwd(qc, kc, vc, out=oc, lse=lse_c, **kw)
        attn.bwd(qc, kc, vc, oc, lse_c, gc, workspace=ws, dq=dqc, dk=dkc, dv=dvc, **kw)
        for dst, src, t in ((o5, oc, Tq), (dq5, dqc, Tq), (dk5, dkc, T), (dv5, dvc, T)):
            dst.copy_(windows(src, t))

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / steps

    t_strided = timed(strided_step)
    same = all(torch.equal(a.permute(0, 2, 1, 3, 4).reshape(b.shape), b)
               for a, b in ((o5, o_ref), (dq5, dq_ref), (dk5, dk_ref), (dv5, dv_ref)))
    same = same and torch.equal(lse_t, lse_ref)
    t_copy = timed(copy_step)
    log(f"[bench] token order: {t_strided:.4f} ms/step in place, {t_copy:.4f} with layout copies")
    return {"ms_per_step": round(t_strided, 5), "with_layout_copies_ms": round(t_copy, 5),
            "steps": steps, "bitwise_equal": bool(same),
            "layout": "K, V in a (B, T, nw, 3, H, d) buffer; Q, dO, O, dQ in (B, Tq, nw, H, d); "
                      "dK, dV in (B, T, nw, 2, H, d)"}


# ---------------------------------------------------------------- CPU oracle

TOLERANCES = {"bf16": (2e-2, 5e-3), "fp16": (2.5e-3, 6.25e-4), "fp32": (1e-5, 1e-5)}


def host_cores() -> int:
    """Cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def oracle_slices(w, host_inputs, budget_s: float, gpu_out, min_slices: int = 1):
    """Run the fp64 oracle on whole (batch, head) slices, one at a time, until
    about ``budget_s`` seconds are spent (at least ``min_slices``), comparing
    those slices of the GPU outputs with it.  Returns (slices done, oracle
    seconds, parity record)."""
    import torch
    from oracle import oracle_bwd, oracle_fwd

    q, k, v, do = host_inputs
    worst = {}
    done, spent = 0, 0.0
    tol = TOLERANCES[w.dtype]
    total_bh = w.B * w.H
    # spread the sampled slices over the batch: first, last, then every 7th
    # index, then the rest, until the time budget is spent
    order = [0, total_bh - 1] + [i for r in range(7) for i in range(r, total_bh, 7)]
    seen = set()
    for idx in order:
        if idx in seen:
            continue
        seen.add(idx)
        b, h = divmod(idx, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        qs, ks, vs, dos = (t[sl].to(torch.float64).numpy() for t in (q, k, v, do))
        t0 = time.perf_counter()
        ro, rl = oracle_fwd(qs, ks, vs, w.scale, w.mask, w.window)
        rdq, rdk, rdv = oracle_bwd(qs, ks, vs, dos, w.scale, w.mask, w.window)
        spent += time.perf_counter() - t0
        done += 1
        for name, ref in (("O", ro), ("dQ", rdq), ("dK", rdk), ("dV", rdv)):
            x = gpu_out[name][sl].double().numpy()
            diff = x - ref
            m = float(np.abs(diff).max())
            r = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
            pm, pr = worst.get(name, (0.0, 0.0))
            worst[name] = (max(pm, m), max(pr, r))
        lerr = float(np.abs(gpu_out["lse"][sl].double().numpy() - rl).max())
        worst["lse_max_abs"] = (max(worst.get("lse_max_abs", (0.0, 0.0))[0], lerr), 0.0)
        if spent >= budget_s and done >= min_slices:
            break
    lse_err = worst.pop("lse_max_abs")[0]
    ok = all(m <= tol[0] and r <= tol[1] for m, r in worst.values())
    parity = {"slices": done, "of": total_bh, "pass": bool(ok),
              "tolerance": {"max_abs": tol[0], "rel_l2": tol[1]},
              "max_abs": {k: round(v[0], 6) for k, v in worst.items()},
              "rel_l2": {k: round(v[1], 7) for k, v in worst.items()},
              "lse_max_abs": round(lse_err, 7)}
    return done, spent, parity


def cpu_baseline(w, host_inputs, pairs_per_bh, budget_s: float, gpu_out):
    """Time the fp64 oracle on whole (batch, head) slices of the workload on
    this host's cores (BLAS threads pinned to them) until about ``budget_s``
    seconds are spent, checking the GPU's outputs of those slices on the way."""
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = host_cores()
    with threadpool_limits(limits=cores, user_api="blas"):
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max([p.get("num_threads", 1) for p in blas] or [1])
        done, spent, parity = oracle_slices(w, host_inputs, budget_s, gpu_out)
    flop_per_bh = 14 * w.d * pairs_per_bh
    base = {
        "value": flop_per_bh * done / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "blas_threads": int(threads),
        "kind": "oracle",
        "sample": (f"{done} of {w.B * w.H} (batch, head) slices of the same workload, "
                   f"fwd+bwd, fp64 NumPy ({blas[0].get('internal_api', '?') if blas else '?'} "
                   f"BLAS, {threads} threads on {cores} cores; elementwise exp "
                   f"single-threaded), {spent:.1f} s"),
    }
    return base, parity


# ------------------------------------------------------------------- a step

class Step:
    """The tensors and calls of one workload's step on the device: inputs,
    outputs and the backward workspace allocated once, then launched kernel
    by kernel (``kernels``) on torch's current stream."""

    def __init__(self, attn, torch, w, host, dev):
        self.attn, self.torch, self.w, self.dev = attn, torch, w, dev
        q, k, v, do = (t.to(dev) for t in host)
        self.iha = None
        if w.P > 1:
            # interleaved head attention: the attention's Q, K, V are the
            # premix outputs (each head's N * P pseudo-tokens) of three
            # [B, N, H, d] inputs; the drawn q, k, v serve only as the first
            # step's values
            self.iha = iha_setup(attn, torch, w, dev)
            q, k, v = (t.view(w.B, w.H, w.Nq, w.d) for t in self.iha["out"])
        self.q, self.k, self.v, self.do = q, k, v, do
        self.o = torch.empty_like(q)
        self.lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        # the larger workspace where it applies: the dQ pass then reads dS kept
        # by the dK/dV pass instead of recomputing S and dP
        self.ws_bytes = attn.binding.workspace_bytes_ds(q, k, mask=w.mask, window=w.window)
        self.kept_ds = self.ws_bytes > attn.binding.workspace_bytes(w.B, w.H, w.Nq)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.kw = dict(mask=w.mask, window=w.window, scale=w.scale)
        self.fused = attn.binding.bwd_fused(q, k, v, mask=w.mask, window=w.window)
        kernels = ("fwd", "bwd") if self.fused else KERNELS
        if self.iha is not None:
            kernels = ("premix",) + kernels + ("premix_bwd",)
        self.kernels = kernels

    def launch(self, kernel):
        attn, iha = self.attn, self.iha
        if kernel == "premix":
            for x, wt, out in zip(iha["x"], iha["w"], iha["out"]):
                attn.binding.premix(x, wt, out=out)
        elif kernel == "premix_bwd":
            for x, wt, g, dx, dw in zip(iha["x"], iha["w"], (self.dq, self.dk, self.dv), iha["dx"],
                                        iha["dw"]):
                attn.binding.premix_bwd(x, wt, g.view(iha["out"][0].shape), dx=dx, dw=dw,
                                        workspace=iha["ws"])
        elif kernel == "fwd":
            attn.fwd(self.q, self.k, self.v, out=self.o, lse=self.lse, **self.kw)
        elif kernel == "bwd":
            attn.bwd(self.q, self.k, self.v, self.o, self.lse, self.do, workspace=self.ws,
                     dq=self.dq, dk=self.dk, dv=self.dv, **self.kw)
        else:
            bit = {"rowsum": attn.binding.PASS_ROWSUM, "dkdv": attn.binding.PASS_DKDV,
                   "dq": attn.binding.PASS_DQ}[kernel]
            attn.bwd(self.q, self.k, self.v, self.o, self.lse, self.do, workspace=self.ws,
                     dq=self.dq, dk=self.dk, dv=self.dv, passes=bit, **self.kw)

    def run(self):
        for kn in self.kernels:
            self.launch(kn)

    def time(self, steps: int, warmup: int):
        """``warmup`` untimed steps, then ``steps`` timed ones between two
        device synchronisations, with HIP events after every kernel (torch
        events on the current stream, the one the kernels run on).  Returns
        (ms per step over the region, mean ms per kernel, p10/median/p90)."""
        torch = self.torch
        for _ in range(warmup):
            self.run()
        torch.cuda.synchronize(self.dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.kernels) + 1)]
              for _ in range(steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(self.dev)
        start.record()
        for s in range(steps):
            ev[s][0].record()
            for i, kn in enumerate(self.kernels):
                self.launch(kn)
                ev[s][i + 1].record()
        stop.record()
        torch.cuda.synchronize(self.dev)
        ms_per_step = start.elapsed_time(stop) / steps
        kern_ms = {kn: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
                   for i, kn in enumerate(self.kernels)}
        return ms_per_step, kern_ms, step_spread(ev, self.kernels)

    def direct_time(self, steps: int) -> float:
        """ms per step of ``steps`` direct steps between two events (no
        per-kernel events): the reference that the autograd and graph timings,
        taken later in the run, are compared with when timed next to it (the
        MFMA-heavy kernels' clock drifts down over a run)."""
        torch = self.torch
        torch.cuda.synchronize(self.dev)
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for _ in range(steps):
            self.run()
        d1.record()
        torch.cuda.synchronize(self.dev)
        return d0.elapsed_time(d1) / steps

    def graph_time(self, replays: int, warm: int = 20) -> float:
        """ms per step of the step captured once in a HIP graph and replayed
        ``replays`` times: the kernels without the host's per-call work.
        ``warm`` untimed replays first: the capture leaves the GPU idle, and
        the MFMA-heavy kernels run up to 25% slower for the first ~20 ms of
        work after an idle spell (traced on the causal workload), as at the
        start of the main region, whose warmup steps absorb it."""
        torch = self.torch
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run()
        for _ in range(warm):
            graph.replay()
        torch.cuda.synchronize(self.dev)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(replays):
            graph.replay()
        g1.record()
        torch.cuda.synchronize(self.dev)
        del graph
        return g0.elapsed_time(g1) / replays

    def outputs(self):
        """A fresh fwd + bwd through attn_fwd / attn_bwd (library-allocated
        outputs), whether it equals the staged step bit for bit, and the
        outputs on the host for the parity check."""
        attn, torch = self.attn, self.torch
        o2, lse2 = attn.fwd(self.q, self.k, self.v, **self.kw)
        dq2, dk2, dv2 = attn.bwd(self.q, self.k, self.v, o2, lse2, self.do, **self.kw)
        torch.cuda.synchronize(self.dev)
        same = all(torch.equal(a, b) for a, b in ((self.o, o2), (self.lse, lse2), (self.dq, dq2),
                                                  (self.dk, dk2), (self.dv, dv2)))
        return same, {"O": o2.cpu(), "lse": lse2.cpu(), "dQ": dq2.cpu(), "dK": dk2.cpu(),
                      "dV": dv2.cpu()}

    def step_label(self):
        if self.fused:
            s = "attn_fwd + attn_bwd (one fused kernel: dK/dV and dQ work side by side)"
        elif self.kept_ds:
            s = "attn_fwd + attn_bwd (row sums, dK/dV keeping dS, dQ = scale dS K)"
        else:
            s = "attn_fwd + attn_bwd (row sums, dK/dV, dQ passes)"
        if self.iha is not None:
            s = ("attn_premix_fwd x3 (Q, K, V pseudo-tokens) + " + s
                 + " over the N * P pseudo-tokens + attn_premix_bwd x3 (dX, dW)")
        return s


def accounting(w, st: Step, ms_per_step: float, kern_ms: dict) -> dict:
    """TFLOP/s of the step, its bound, and the dominant kernel's roofline."""
    pairs_bh = visible_pairs(w.mask, w.window, w.Nq, w.Nk)
    sw = step_work(w, pairs_bh)
    work = kernel_work(w, pairs_bh, st.kept_ds)
    value = sw["flops"] / (ms_per_step * 1e-3) / 1e12
    dom = max(st.kernels, key=lambda kn: kern_ms[kn])
    wk = work[dom]
    roof = kernel_roofline(wk, sw["bound"], sw["peak"], kern_ms[dom])
    traffic = stored_traffic(w.name, dom)
    if roof is None:
        roof = {"bound": "latency", "achieved": None, "peak": None, "unit": None, "frac": None}
    # measured traffic against what the kernel must move: the method's bytes
    # plus this library's workspace (kept dS) where it uses one
    roof.update(traffic=traffic, kernel=dom,
                algorithmic_per_launch={"flops": wk["flops"], "bytes": wk["bytes"]},
                workspace_bytes_per_launch=wk["workspace_bytes"],
                traffic_over_algorithmic_plus_workspace=(
                    round(traffic / (wk["bytes"] + wk["workspace_bytes"]), 4) if traffic else None))
    return {"pairs_bh": pairs_bh, "pairs": pairs_bh * w.B * w.H, "step": sw, "work": work,
            "value": value, "dom": dom, "roofline": roof,
            "step_roofline_frac": round(sw["roofline_ms"] / ms_per_step, 4)}


def shape_of(w) -> dict:
    return {"B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "mask": w.mask,
            "window": w.window, "dtype": w.dtype}


# the benchmark configurations, in order: the exact fp32 check, the Hiera
# mask-unit windows, the Hiera global stage, the causal LM, the causal sliding
# window over pseudo-heads
CONFIGS = ("tiny_exact_fp32", "block_local_hiera", "global_vision", "causal_lm",
           "sliding_pseudo_head")


def config_entry(attn, torch, w, dev, steps: int, warmup: int, parity_s: float) -> dict:
    """One configuration measured on its own: timed steps, accounting, and
    sampled-slice parity against the oracle (outside the timed region)."""
    from head_attention_attn_amd.inputs import workload_inputs

    host = workload_inputs(w, seed=0)
    st = Step(attn, torch, w, host, dev)
    if w.dtype == "fp32":
        # a step of a few microseconds: more steps for a stable median
        steps, warmup = steps * 10, warmup * 10
    ms, kern_ms, spread = st.time(steps, warmup)
    graph_ms = st.graph_time(steps)
    acc = accounting(w, st, ms, kern_ms)
    same, gpu_out = st.outputs()
    _, _, parity = oracle_slices(w, host, parity_s, gpu_out)
    parity["staged_equals_attn_bwd"] = bool(same)
    entry = {"workload": w.name, "shape": shape_of(w), "step": st.step_label(),
             "bound": acc["step"]["bound"], "steps": steps,
             "ms_per_step": round(ms, 5), "spread": spread,
             "tflops": round(acc["value"], 3),
             "pct_of_bf16_mfma_peak": round(100 * acc["value"] / MFMA_BF16_PEAK_TFLOPS, 3),
             "step_roofline_ms": round(acc["step"]["roofline_ms"], 5),
             "step_roofline_frac": acc["step_roofline_frac"],
             "per_kernel_ms": {kn: round(kern_ms[kn], 5) for kn in st.kernels},
             "hip_graph_ms_per_step": round(graph_ms, 5),
             "dominant": acc["roofline"], "parity": parity}
    log(f"[bench] config {w.name}: {ms:.4f} ms/step, {acc['value']:.1f} TFLOP/s, "
        f"{acc['dom']} frac {acc['roofline'].get('frac')}, parity "
        f"{'pass' if parity['pass'] else 'FAIL'} ({parity['slices']} slices)")
    del st
    torch.cuda.empty_cache()
    return entry


# --------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="causal_lm")
    ap.add_argument("--dtype", choices=("bf16", "fp16"), default=None,
                    help="run a 16-bit workload in this element type instead")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU-oracle baseline (0 skips it)")
    ap.add_argument("--configs", default="all",
                    help="'all' (every benchmark configuration, each timed and checked on "
                         "its own after the headline workload), 'none', or a comma list")
    ap.add_argument("--config-parity-seconds", type=float, default=3.0,
                    help="oracle time budget of each configuration's sampled-slice parity")
    ap.add_argument("--graph-steps", type=int, default=20,
                    help="steps replayed from the step captured in a HIP graph (0: skip)")
    ap.add_argument("--autograd-steps", type=int, default=20,
                    help="after the timed region, time this many steps through the "
                         "torch.autograd wrapper (0 skips it)")
    ap.add_argument("--layout-steps", type=int, default=20,
                    help="block mask only: after the timed region, time this many steps "
                         "with every tensor in Hiera's token order (strided entry points), "
                         "and the same step done by copying to and from the contiguous "
                         "layout (0 skips it)")
    ap.add_argument("--cold-steps", type=int, default=50,
                    help="after the timed region, time this many steps each preceded by "
                         "a read of --flush-mib MiB that evicts the inputs from the L2 "
                         "and the Infinity Cache (0 skips it)")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="size of the cache-evicting read before each cold step")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run a plain device copy of this "
                         "many MiB 5 times (a known-size reference for HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): "
              "the attention path is not sharded across GPUs", file=sys.stderr)
        return 2

    import torch
    import head_attention_attn_amd as attn
    from head_attention_attn_amd.inputs import WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    w = WORKLOADS[args.workload]
    if args.dtype is not None:
        if (w.dtype == "fp32") != (args.dtype == "fp32"):
            log("--dtype switches between the 16-bit types only")
            return 2
        w = dataclasses.replace(w, dtype=args.dtype)
    if args.configs == "all":
        config_names = list(CONFIGS)
    elif args.configs == "none":
        config_names = []
    else:
        config_names = [c for c in args.configs.split(",") if c]
        unknown = [c for c in config_names if c not in WORKLOADS]
        if unknown:
            log(f"unknown configuration(s): {unknown}")
            return 2
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"[bench] {w} on {props.name} ({getattr(props, 'gcnArchName', '?')}, "
        f"{props.multi_processor_count} CUs)")

    host = workload_inputs(w, seed=0)
    st = Step(attn, torch, w, host, dev)
    kernels = st.kernels
    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps of {', '.join(kernels)}")
    K = args.steps
    ms_per_step, kern_ms, warm_spread = st.time(K, args.warmup)
    log(f"[bench] {ms_per_step:.4f} ms/step; per kernel (ms): "
        + ", ".join(f"{kn} {kern_ms[kn]:.4f}" for kn in kernels))

    # the same step through the autograd wrapper (forward, then backward from
    # dO by torch.autograd.grad), timed after the main region between two
    # blocks of direct steps, its ratio taken against their mean
    autograd_rec = None
    if args.autograd_steps > 0:
        qa, ka, va = (t.detach().requires_grad_(True) for t in (st.q, st.k, st.v))

        def ag_step():
            oa = attn.fused_attention(qa, ka, va, w.mask, w.window, w.scale)
            return torch.autograd.grad(oa, (qa, ka, va), st.do)

        if st.iha is not None:
            # the whole interleaved-head step: premix, attention, both backwards
            leaves = [t.detach().requires_grad_(True) for t in st.iha["x"] + st.iha["w"]]

            def ag_step():
                oa = attn.iha_attention(*leaves, window=w.window, scale=w.scale)
                return torch.autograd.grad(oa, leaves, st.do)

        for _ in range(3):
            ag_step()
        before = st.direct_time(args.autograd_steps)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(args.autograd_steps):
            ag_step()
        a1.record()
        torch.cuda.synchronize(dev)
        ag_ms = a0.elapsed_time(a1) / args.autograd_steps
        adjacent = 0.5 * (before + st.direct_time(args.autograd_steps))
        autograd_rec = {"ms_per_step": round(ag_ms, 5), "steps": args.autograd_steps,
                        "adjacent_direct_ms_per_step": round(adjacent, 5),
                        "over_direct_calls": round(ag_ms / adjacent, 4)}
        log(f"[bench] autograd wrapper: {ag_ms:.4f} ms/step")
        del qa, ka, va

    # the same step captured once in a HIP graph and replayed: the kernels
    # without the host's per-call launch work (every call takes preallocated
    # outputs and workspace, so the capture allocates nothing); its ratio is
    # taken against direct steps timed just before and after the replays
    graph_rec = None
    if args.graph_steps > 0:
        before = st.direct_time(args.graph_steps)
        g_ms = st.graph_time(args.graph_steps)
        adjacent = 0.5 * (before + st.direct_time(args.graph_steps))
        graph_rec = {"ms_per_step": round(g_ms, 5), "steps": args.graph_steps,
                     "adjacent_direct_ms_per_step": round(adjacent, 5),
                     "over_direct_calls": round(g_ms / adjacent, 4)}
        log(f"[bench] HIP graph replay: {g_ms:.4f} ms/step")

    # cache-flushed steps: before each, a read of a buffer four times the
    # 256 MB Infinity Cache evicts Q, K, V, dO (and the previous step's
    # outputs) from every cache, so the forward reads them from HBM.  A read,
    # not a write: a write would leave the caches full of dirty lines whose
    # write-back the next kernel would pay for (measured: the block-local
    # forward 0.049 -> 0.102 ms after a 1 GiB fill)
    cold_rec = None
    if args.cold_steps > 0:
        flush = torch.ones(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)]
               for _ in range(args.cold_steps)]
        torch.cuda.synchronize(dev)
        for s in range(args.cold_steps):
            torch.sum(flush, dim=0, out=sink)
            cev[s][0].record()
            for i, kn in enumerate(kernels):
                st.launch(kn)
                cev[s][i + 1].record()
        torch.cuda.synchronize(dev)
        cold_rec = step_spread(cev, kernels)
        cold_rec.update(steps=args.cold_steps, flush_mib=args.flush_mib)
        log(f"[bench] cache-flushed steps: median {cold_rec['ms_per_step']['median']:.4f} ms/step")
        del flush, sink

    layout_rec = None
    if args.layout_steps > 0 and w.mask == "block":
        layout_rec = token_order_timing(attn, torch, w, st.q, st.k, st.v, st.do, st.ws, st.kw,
                                        st.fused, st.o, st.lse, st.dq, st.dk, st.dv,
                                        args.layout_steps, dev)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        log(f"[bench] copy calibration: 5 copies of {args.copy_calibration_mib} MiB")
        del src, dst

    # ---- accounting
    acc = accounting(w, st, ms_per_step, kern_ms)
    value, dom, roof = acc["value"], acc["dom"], acc["roofline"]
    wk = acc["work"][dom]
    bound, peak = acc["step"]["bound"], acc["step"]["peak"]
    # the dominant kernel at the clock it ran at in the stored counter run
    # (the MFMA peak is quoted at 2.4 GHz; MFMA-heavy kernels run slower under
    # their own power draw).  Approximate: GRBM_GUI_ACTIVE, which gives the
    # clock, reads up to a few per cent high.
    clk = stored_clock(w.name, dom)
    clock_rec = None
    if clk is not None:
        clock_rec = {"kernel": dom, "ghz": clk, "source": f"profiles/mfma_{w.name}.txt"}
        if bound in ("mfma", "alu"):
            clock_rec["kernel_frac_of_peak_at_clock_approx"] = round(
                wk["flops"] / (kern_ms[dom] * 1e-3) / 1e12 / (peak * clk / 2.4), 4)
    timing = {"warm": warm_spread, "cache_flushed": cold_rec}
    for rec_t in timing.values():
        if rec_t is not None:
            r = kernel_roofline(wk, bound, peak, rec_t["per_kernel_ms"][dom]["median"])
            rec_t["roofline_frac_at_median"] = None if r is None else r["frac"]

    # ---- outputs for the parity check (a full fwd + bwd through attn_bwd)
    same, gpu_out = st.outputs()
    cpu = None
    parity = {"staged_equals_attn_bwd": bool(same)}
    if st.iha is not None:
        # the attention's inputs are the premix outputs
        host = tuple(t.cpu() for t in (st.q, st.k, st.v)) + (host[3],)
        parity["premix_error_over_bound"] = round(premix_parity(st.iha, w), 4)
    if args.cpu_seconds > 0:
        log(f"[bench] timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        cpu, par = cpu_baseline(w, host, acc["pairs_bh"], args.cpu_seconds, gpu_out)
        parity.update(par)

    cfg = {"workload": w.name, **shape_of(w), "visible_pairs": acc["pairs"],
           "workspace_bytes": st.ws_bytes, "step": st.step_label(),
           "bound": bound, "arithmetic_intensity": acc["step"]["arithmetic_intensity"]}
    if st.iha is not None:
        cfg.update(P=w.P, tokens=w.Nq // w.P)
    headline = {"ms_per_step": round(ms_per_step, 5), "spread": warm_spread,
                "per_kernel_ms": {kn: round(kern_ms[kn], 5) for kn in kernels},
                "tflops": round(value, 3), "dominant": roof, "parity": parity}
    del st, gpu_out
    torch.cuda.empty_cache()

    # ---- every benchmark configuration, each on its own
    configs = []
    for name in config_names:
        cw = WORKLOADS[name]
        if args.dtype is not None and cw.dtype != "fp32":
            cw = dataclasses.replace(cw, dtype=args.dtype)
        if cw == w and args.cpu_seconds > 0:
            # the headline workload: its measurement above
            configs.append({"workload": w.name, "shape": shape_of(w), "step": cfg["step"],
                            "bound": bound, "steps": K,
                            "ms_per_step": headline["ms_per_step"], "spread": warm_spread,
                            "tflops": headline["tflops"],
                            "pct_of_bf16_mfma_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 3),
                            "step_roofline_ms": round(acc["step"]["roofline_ms"], 5),
                            "step_roofline_frac": acc["step_roofline_frac"],
                            "per_kernel_ms": headline["per_kernel_ms"],
                            "hip_graph_ms_per_step": graph_rec and graph_rec["ms_per_step"],
                            "dominant": roof, "parity": parity})
            continue
        configs.append(config_entry(attn, torch, cw, dev, max(K // 4, 20), max(args.warmup // 4, 3),
                                    args.config_parity_seconds))

    rec = {
        "metric": "attention fwd+bwd TFLOP/s at 1 MI355X; % of bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic i.i.d. N(0,1) Q, K, V, dO (seed 0), resident in HBM",
        "config": cfg,
        "pct_of_bf16_mfma_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 3),
        "step_roofline_frac": acc["step_roofline_frac"],
        "measured_clock": clock_rec,
        "per_kernel_ms": headline["per_kernel_ms"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "configs": configs,
        "autograd": autograd_rec,
        "timing": timing,
        "hip_graph": graph_rec,
        "token_order": layout_rec,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "cus": props.multi_processor_count, "torch": torch.__version__,
                   "hip": torch.version.hip},
    }
    print(json.dumps(rec), flush=True)
    ok = same and parity.get("pass", True) and (layout_rec is None or layout_rec["bitwise_equal"])
    ok = ok and parity.get("premix_error_over_bound", 0.0) <= 1.0
    ok = ok and all(c["parity"]["pass"] and c["parity"].get("staged_equals_attn_bwd", True)
                    for c in configs)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
