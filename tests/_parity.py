"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd.inputs import make_inputs
from oracle import oracle_bwd, oracle_fwd

# Tolerances, per tensor over the whole compared set: max |x - y| and
# ||x - y||_2 / ||y||_2.  bf16 inputs: 2e-2 and 5e-3; fp32 inputs: 1e-5 both.
# lse (not graded): 1e-3 (bf16), 1e-5 (fp32), absolute.  fp16 inputs: the
# bf16 bounds times the ratio of the two unit roundoffs, 2^-11 / 2^-8 = 1/8
# (every error term of the 16-bit path -- P and dS rounded to the input type
# before their products, outputs rounded -- scales with it).
TOL = {"bf16": (2e-2, 5e-3, 1e-3), "fp16": (2.5e-3, 6.25e-4, 1.25e-4),
       "fp32": (1e-5, 1e-5, 1e-5)}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def errors(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = x - ref
    maxabs = float(np.max(np.abs(d))) if d.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / nrm) if nrm > 0 else float(np.linalg.norm(d))
    return maxabs, rel


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_fwd_bwd(q, k, v, do, mask, window, scale, keep_ds=True):
    dev = "cuda"
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = attn.fwd(qd, kd, vd, mask=mask, window=window, scale=scale)
    dq, dk, dv = attn.bwd(qd, kd, vd, o, lse, dod, mask=mask, window=window, scale=scale,
                          keep_ds=keep_ds)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def compare(name_vals, dtype, label="", tol=None, abs_only=(), amax_rel=0.0):
    """name_vals: list of (name, gpu ndarray, oracle ndarray).  Asserts the
    tolerance (``tol`` = (max-abs, rel-L2, lse) overrides the dtype's) and
    returns a dict of errors.  Tensors named in ``abs_only`` are exactly zero
    in exact arithmetic, where rel-L2 is undefined: only max-abs is checked.
    ``amax_rel`` widens each tensor's max-abs bound by amax_rel * max|ref|
    (the output rounding of large-magnitude results)."""
    amax, rel, lse_tol = TOL[dtype] if tol is None else tol
    report = {}
    for name, x, ref in name_vals:
        if name == "lse":
            fin = np.isfinite(ref)
            assert np.array_equal(fin, np.isfinite(x)), f"{label} lse -inf pattern differs"
            assert np.all(np.isneginf(x[~fin])), f"{label} lse of empty rows must be -inf"
            m, _ = errors(x[fin], ref[fin]) if fin.any() else (0.0, 0.0)
            report[name] = (m, None)
            assert m <= lse_tol, f"{label} lse max-abs {m:.3e} > {lse_tol}"
            continue
        m, r = errors(x, ref)
        report[name] = (m, r)
        assert np.all(np.isfinite(x)), f"{label} {name} has non-finite values"
        bound = amax + amax_rel * (float(np.abs(ref).max()) if ref.size else 0.0)
        assert m <= bound, f"{label} {name} max-abs {m:.3e} > {bound:.3e}"
        if name in abs_only:
            continue
        assert r <= rel, f"{label} {name} rel-L2 {r:.3e} > {rel}"
    return report


def parity_case(B, H, Nq, Nk, d, dtype, mask, window=0, seed=0, scale=None, transform=None,
                tol=None, abs_only=(), amax_rel=0.0, keep_ds=True):
    """Full-tensor parity of one small case; returns the error report.
    ``keep_ds`` picks the backward workspace: large enough for the dQ pass to
    read dS kept by the dK/dV pass (where that path applies), or the minimum
    (dQ recomputes S and dP)."""
    scale = float(torch.tensor(1.0 / np.sqrt(d), dtype=torch.float32)) if scale is None else scale
    say(f"[parity] B={B} H={H} Nq={Nq} Nk={Nk} d={d} {dtype} mask={mask} W={window} seed={seed}"
        f" keep_ds={keep_ds}")
    q, k, v, do = make_inputs(B, H, Nq, Nk, d, dtype, seed)
    if transform is not None:
        q, k, v, do = transform(q, k, v, do)
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, mask, window, scale, keep_ds=keep_ds)
    ro, rl = oracle_fwd(to64(q), to64(k), to64(v), scale, mask, window)
    rdq, rdk, rdv = oracle_bwd(to64(q), to64(k), to64(v), to64(do), scale, mask, window)
    return compare([("O", to64(o), ro), ("lse", to64(lse), rl), ("dQ", to64(dq), rdq),
                    ("dK", to64(dk), rdk), ("dV", to64(dv), rdv)], dtype,
                   label=f"B{B}H{H}N{Nq}x{Nk}d{d}{dtype}{mask}{window}", tol=tol,
                   abs_only=abs_only, amax_rel=amax_rel)
