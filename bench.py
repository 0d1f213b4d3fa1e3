"""Throughput of fused attention forward + backward on one MI355X.

One step = the whole hot path over one batch of synthetic input already
resident in HBM: ``attn_fwd`` (O and lse), then the three backward passes
(row sums D, dK/dV, dQ) through ``attn_bwd_passes``, all on torch's current
stream.  W untimed warmup steps, then K timed steps bracketed by a device
synchronisation on both sides.  HIP events recorded between the calls give
each kernel's average duration over the timed region.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value      algorithmic TFLOP/s of the step: (4 d + 10 d) flops per visible
             (query, key) pair (forward 4 d, backward 10 d) over the step time
  roofline   the kernel with the largest share of the step, its algorithmic
             bytes (HBM-bound) or flops (MFMA-bound) per launch over its
             measured average duration, against the MI355X peak; ``traffic``
             is the HBM bytes per launch that rocprofv3 counters measured for
             that kernel (profiles/traffic_<workload>.txt), or null when the
             kernel sources changed since
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
             workload on this host, in the same unit
  parity     GPU outputs of the sampled slices against the oracle, checked
             outside the timed region
  timing     p10 / median / p90 of the step and of each kernel over the timed
             steps ("warm": back to back) and over steps each preceded by a
             1 GiB read that evicts every cache ("cache_flushed"), with the
             dominant kernel's roofline fraction at each median

Workloads (``--workload``): block_local_hiera (default; Hiera-Base mask-unit
attention, 49 windows of 64 tokens, B=128, d=96), block_pooled_hiera (the
same windows with 16 pooled query rows each, H=2), global_vision, causal_lm,
sliding_pseudo_head, tiny_exact_fp32.  ``--gpus`` above 1 is refused: this
path runs on one GPU.
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
    fused single-tile backward is credited with.  Bytes: every tensor the
    kernel must read or write, once.  With ``kept_ds`` the dK/dV pass also
    writes dS (bf16, 2 bytes per visible pair) and the dQ pass reads dS and K
    only, instead of Q, dO, lse, D, K and V."""
    es = 4 if w.dtype == "fp32" else 2
    bh = w.B * w.H
    q_rows, k_rows, d = bh * w.Nq, bh * w.Nk, w.d
    pairs = bh * pairs_per_bh
    ds_bytes = 2 * pairs if kept_ds else 0
    dq_bytes = ((q_rows * d + k_rows * d) * es + ds_bytes if kept_ds
                else (3 * q_rows * d + 2 * k_rows * d) * es + 8 * q_rows)
    return {
        "fwd": dict(flops=4 * d * pairs,
                    bytes=(2 * q_rows * d + 2 * k_rows * d) * es + 4 * q_rows),
        "rowsum": dict(flops=2 * d * q_rows, bytes=2 * q_rows * d * es + 4 * q_rows),
        "dkdv": dict(flops=8 * d * pairs,
                     bytes=(2 * q_rows * d + 4 * k_rows * d) * es + 8 * q_rows + ds_bytes),
        "dq": dict(flops=2 * d * pairs, bytes=dq_bytes),
        # the fused single-tile backward: reads Q, K, V, dO, lse, writes dQ,
        # dK, dV (its row sums come from P and dP in-tile, O is not read)
        "bwd": dict(flops=10 * d * pairs,
                    bytes=(3 * q_rows * d + 4 * k_rows * d) * es + 4 * q_rows),
    } | premix_work(w, es)


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

def cpu_baseline(w, host_inputs, pairs_per_bh, budget_s: float, gpu_out):
    """Time the fp64 oracle on whole (batch, head) slices, one at a time, until
    about ``budget_s`` seconds are spent; compare those slices of the GPU
    outputs with the oracle's while at it."""
    import torch
    from threadpoolctl import threadpool_info
    from oracle import oracle_bwd, oracle_fwd

    q, k, v, do = host_inputs
    flop_per_bh = 14 * w.d * pairs_per_bh
    worst = {}
    done, spent = 0, 0.0
    tol = {"bf16": (2e-2, 5e-3), "fp16": (2.5e-3, 6.25e-4), "fp32": (1e-5, 1e-5)}[w.dtype]
    total_bh = w.B * w.H
    # spread the sampled slices over the batch: first, last, then every 7th
    # index, then the rest, until the time budget is spent
    order = [0, total_bh - 1] + [i for r in range(7) for i in range(r, total_bh, 7)]
    seen = []
    for idx in order:
        if idx in seen:
            continue
        seen.append(idx)
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
        if spent >= budget_s:
            break
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    base = {
        "value": flop_per_bh * done / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{done} of {total_bh} (batch, head) slices of the same workload, "
                   f"fwd+bwd, fp64 NumPy ({blas[0].get('internal_api', '?') if blas else '?'} "
                   f"BLAS, {threads} threads; elementwise exp single-threaded), "
                   f"{spent:.1f} s"),
    }
    ok = all(m <= tol[0] and r <= tol[1] for m, r in worst.values())
    parity = {"slices": done, "pass": bool(ok),
              "max_abs": {k: round(v[0], 6) for k, v in worst.items()},
              "rel_l2": {k: round(v[1], 7) for k, v in worst.items()}}
    return base, parity


# --------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="block_local_hiera")
    ap.add_argument("--dtype", choices=("bf16", "fp16"), default=None,
                    help="run a 16-bit workload in this element type instead")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU-oracle baseline (0 skips it)")
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
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"[bench] {w} on {props.name} ({getattr(props, 'gcnArchName', '?')}, "
        f"{props.multi_processor_count} CUs)")

    host = workload_inputs(w, seed=0)
    q, k, v, do = (t.to(dev) for t in host)
    iha = None
    if w.P > 1:
        # interleaved head attention: the attention's Q, K, V are the premix
        # outputs (each head's N * P pseudo-tokens) of three [B, N, H, d]
        # inputs; the drawn q, k, v serve only as the first step's values
        iha = iha_setup(attn, torch, w, dev)
        q, k, v = (t.view(w.B, w.H, w.Nq, w.d) for t in iha["out"])
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # the larger workspace where it applies: the dQ pass then reads dS kept by
    # the dK/dV pass instead of recomputing S and dP
    ws_bytes = attn.binding.workspace_bytes_ds(q, k, mask=w.mask, window=w.window)
    kept_ds = ws_bytes > attn.binding.workspace_bytes(w.B, w.H, w.Nq)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    kw = dict(mask=w.mask, window=w.window, scale=w.scale)

    fused = attn.binding.bwd_fused(q, k, v, mask=w.mask, window=w.window)
    kernels = ("fwd", "bwd") if fused else KERNELS
    if iha is not None:
        kernels = ("premix",) + kernels + ("premix_bwd",)

    def launch(kernel):
        if kernel == "premix":
            for x, wt, out in zip(iha["x"], iha["w"], iha["out"]):
                attn.binding.premix(x, wt, out=out)
        elif kernel == "premix_bwd":
            for x, wt, g, dx, dw in zip(iha["x"], iha["w"], (dq, dk, dv), iha["dx"], iha["dw"]):
                attn.binding.premix_bwd(x, wt, g.view(iha["out"][0].shape), dx=dx, dw=dw,
                                        workspace=iha["ws"])
        elif kernel == "fwd":
            attn.fwd(q, k, v, out=o, lse=lse, **kw)
        elif kernel == "bwd":
            attn.bwd(q, k, v, o, lse, do, workspace=ws, dq=dq, dk=dk, dv=dv, **kw)
        else:
            bit = {"rowsum": attn.binding.PASS_ROWSUM, "dkdv": attn.binding.PASS_DKDV,
                   "dq": attn.binding.PASS_DQ}[kernel]
            attn.bwd(q, k, v, o, lse, do, workspace=ws, dq=dq, dk=dk, dv=dv, passes=bit, **kw)

    for _ in range(args.warmup):
        for kn in kernels:
            launch(kn)
    torch.cuda.synchronize(dev)
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)]
          for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    start.record()
    for s in range(K):
        ev[s][0].record()
        for i, kn in enumerate(kernels):
            launch(kn)
            ev[s][i + 1].record()
    stop.record()
    torch.cuda.synchronize(dev)
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / K
    kern_ms = {kn: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K)) / K
               for i, kn in enumerate(kernels)}
    warm_spread = step_spread(ev, kernels)
    log(f"[bench] {ms_per_step:.4f} ms/step; per kernel (ms): "
        + ", ".join(f"{kn} {kern_ms[kn]:.4f}" for kn in kernels))

    # the same step through the autograd wrapper (forward, then backward from
    # dO by torch.autograd.grad), timed on its own after the main region
    autograd_rec = None
    if args.autograd_steps > 0:
        qa, ka, va = (t.detach().requires_grad_(True) for t in (q, k, v))

        def ag_step():
            oa = attn.fused_attention(qa, ka, va, w.mask, w.window, w.scale)
            return torch.autograd.grad(oa, (qa, ka, va), do)

        if iha is not None:
            # the whole interleaved-head step: premix, attention, both backwards
            leaves = [t.detach().requires_grad_(True) for t in iha["x"] + iha["w"]]

            def ag_step():
                oa = attn.iha_attention(*leaves, window=w.window, scale=w.scale)
                return torch.autograd.grad(oa, leaves, do)

        for _ in range(3):
            ag_step()
        torch.cuda.synchronize(dev)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(args.autograd_steps):
            ag_step()
        a1.record()
        torch.cuda.synchronize(dev)
        ag_ms = a0.elapsed_time(a1) / args.autograd_steps
        autograd_rec = {"ms_per_step": round(ag_ms, 5), "steps": args.autograd_steps,
                        "over_direct_calls": round(ag_ms / ms_per_step, 4)}
        log(f"[bench] autograd wrapper: {ag_ms:.4f} ms/step")
        del qa, ka, va

    # the same step captured once in a HIP graph and replayed: the kernels
    # without the host's per-call launch work (every call takes preallocated
    # outputs and workspace, so the capture allocates nothing)
    graph_rec = None
    if args.graph_steps > 0:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for kn in kernels:
                launch(kn)
        graph.replay()
        torch.cuda.synchronize(dev)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.graph_steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize(dev)
        g_ms = g0.elapsed_time(g1) / args.graph_steps
        graph_rec = {"ms_per_step": round(g_ms, 5), "steps": args.graph_steps,
                     "over_direct_calls": round(g_ms / ms_per_step, 4)}
        log(f"[bench] HIP graph replay: {g_ms:.4f} ms/step")
        del graph

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
                launch(kn)
                cev[s][i + 1].record()
        torch.cuda.synchronize(dev)
        cold_rec = step_spread(cev, kernels)
        cold_rec.update(steps=args.cold_steps, flush_mib=args.flush_mib)
        log(f"[bench] cache-flushed steps: median {cold_rec['ms_per_step']['median']:.4f} ms/step")
        del flush, sink

    layout_rec = None
    if args.layout_steps > 0 and w.mask == "block":
        layout_rec = token_order_timing(attn, torch, w, q, k, v, do, ws, kw, fused, o, lse, dq, dk,
                                        dv, args.layout_steps, dev)

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
    pairs_bh = visible_pairs(w.mask, w.window, w.Nq, w.Nk)
    pairs = pairs_bh * w.B * w.H
    flops_step = 14 * w.d * pairs
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    work = kernel_work(w, pairs_bh, kept_ds)
    dom = max(kernels, key=lambda kn: kern_ms[kn])
    wk = work[dom]
    ai = wk["flops"] / wk["bytes"]
    if w.dtype in ("bf16", "fp16"):
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        mfma_bound = ai >= ridge
        peak_c, bound_c = MFMA_BF16_PEAK_TFLOPS, "mfma"
    else:
        ridge = FP32_VECTOR_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        mfma_bound = ai >= ridge
        peak_c, bound_c = FP32_VECTOR_PEAK_TFLOPS, "alu"
    t_dom = kern_ms[dom] * 1e-3
    traffic = stored_traffic(w.name, dom)
    if mfma_bound:
        achieved = wk["flops"] / t_dom / 1e12
        roof = {"bound": bound_c, "achieved": round(achieved, 2), "peak": peak_c,
                "unit": "TFLOP/s", "frac": round(achieved / peak_c, 4)}
    else:
        achieved = wk["bytes"] / t_dom / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = {"flops": wk["flops"], "bytes": wk["bytes"]}
    # the peak at the clock the dominant kernel ran at under load (the MFMA
    # peak is quoted at 2.4 GHz; MFMA-heavy kernels run at 1.8-2.1 GHz)
    clk = stored_clock(w.name, dom)
    clock_rec = None if clk is None else {
        "kernel": dom, "ghz": clk, "source": f"profiles/mfma_{w.name}.txt",
        "pct_of_bf16_mfma_peak_at_clock": round(100 * value / (MFMA_BF16_PEAK_TFLOPS * clk / 2.4), 3)}
    timing = {"warm": warm_spread, "cache_flushed": cold_rec}
    for rec_t in timing.values():
        if rec_t is not None:
            # the dominant kernel's median duration against its roofline
            t_med = rec_t["per_kernel_ms"][dom]["median"] * 1e-3
            rec_t["roofline_frac_at_median"] = round(
                (wk["flops"] / t_med / 1e12 / peak_c) if mfma_bound
                else (wk["bytes"] / t_med / 1e9 / HBM_PEAK_GBS), 4)

    # ---- outputs for the parity check (a full fwd + bwd through attn_bwd)
    o2, lse2 = attn.fwd(q, k, v, **kw)
    dq2, dk2, dv2 = attn.bwd(q, k, v, o2, lse2, do, **kw)
    torch.cuda.synchronize(dev)
    same = all(torch.equal(a, b) for a, b in ((o, o2), (lse, lse2), (dq, dq2), (dk, dk2),
                                              (dv, dv2)))
    gpu_out = {"O": o2.cpu(), "dQ": dq2.cpu(), "dK": dk2.cpu(), "dV": dv2.cpu()}

    cpu = None
    parity = {"staged_equals_attn_bwd": bool(same)}
    if iha is not None:
        # the attention's inputs are the premix outputs
        host = tuple(t.cpu() for t in (q, k, v)) + (host[3],)
        parity["premix_error_over_bound"] = round(premix_parity(iha, w), 4)
    if args.cpu_seconds > 0:
        log(f"[bench] timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        cpu, par = cpu_baseline(w, host, pairs_bh, args.cpu_seconds, gpu_out)
        parity.update(par)

    cfg = {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
           "mask": w.mask, "window": w.window, "dtype": w.dtype,
           "visible_pairs": pairs,
           "workspace_bytes": ws_bytes,
           "step": ("attn_fwd + attn_bwd (one fused kernel: dK/dV and dQ waves side by side)"
                    if fused else
                    "attn_fwd + attn_bwd (row sums, dK/dV keeping dS, dQ = scale dS K)"
                    if kept_ds else "attn_fwd + attn_bwd (row sums, dK/dV, dQ passes)")}
    if iha is not None:
        cfg.update(P=w.P, tokens=w.Nq // w.P,
                   step="attn_premix_fwd x3 (Q, K, V pseudo-tokens) + " + cfg["step"]
                        + " over the N * P pseudo-tokens + attn_premix_bwd x3 (dX, dW)")
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
        "measured_clock": clock_rec,
        "per_kernel_ms": {kn: round(kern_ms[kn], 5) for kn in kernels},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
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
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
