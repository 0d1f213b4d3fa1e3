"""Seeded synthetic inputs for the attention path.

This module holds no attention arithmetic: it only names the workloads and
draws their inputs, so that the HIP library and the fp64 oracle are fed the
very same values.  Recipe: one CPU ``torch.Generator`` seeded with ``seed``;
Q, K, V, dO drawn in that order with ``torch.randn(shape, float32)``; for bf16
workloads each tensor is then rounded to bfloat16 (fp16 workloads: float16),
round to nearest even.
The oracle widens exactly these values to float64.

Workloads (shapes after the pages' own models; the activations themselves
are synthetic i.i.d. N(0, 1)):

* tiny_exact_fp32 -- a small exact-check case the oracle finishes instantly.
* block_local_hiera -- Hiera-style mask-unit attention at the first stage of
  a 224x224 input: a 56x56 = 3136-token grid split into 49 independent
  windows of 64 contiguous tokens, batch 128 ("hiera-optim 0.1.0", Results:
  Hiera-Base 224x224, B=128; sdist mask_unit.py: windows as independent
  batches).
* block_pooled_hiera -- the mask-unit block where Hiera pools its queries
  (hiera-optim sdist mask_unit.py, ``MaskUnitAttentionFast.forward`` with
  ``q_stride`` = 4; the module docstring names the pooled stage's T = 16):
  the 3136 keys of the 56x56 grid in 49 windows of 64, each window holding
  64 / 4 = 16 max-pooled query rows, so Nq = 784.  The stage's width doubles
  (hierarchical encoders: embed_dim * 2^stage) and so do its heads, leaving
  head_dim = 96: B=128, H=2, d=96.  Windows are contiguous runs here (the
  permute that makes them contiguous is the caller's).
* global_vision -- Hiera's global-attention stage on a 14x14 grid.
* causal_lm -- causal attention of a 20-head, d=128 LLaMA at N=8192
  ("IHA-CUDA", End-to-End Training Benchmark).
* sliding_pseudo_head -- causal sliding window W = 1024 (WSL = 1023) over
  20 heads x 4 pseudo-heads at N=4096 ("IHA-CUDA", FLOP Matching).
* iha_joint -- interleaved head attention with the joint softmax: the
  20-head d=128 LLaMA at N = 8192 tokens, P = 4 pseudo-heads built by the
  premix from Q, K, V (W ~ N(0, 1/H)), and one causal sliding window of
  W = WSL + 1 = 1024 pseudo-tokens over each head's 32768 pseudo-tokens
  ("IHA-CUDA", End-to-End Training Benchmark and FLOP Matching, N = 8192
  row).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str          # "bf16", "fp16" or "fp32"
    mask: str           # "none" | "causal" | "sliding" | "block"
    window: int = 0
    P: int = 1          # IHA pseudo-heads: Nq = Nk = N * P pseudo-tokens built by the premix

    @property
    def scale(self) -> float:
        """1/sqrt(d) as the fp32 value handed to both sides."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    def as_dict(self) -> dict:
        return asdict(self)


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_exact_fp32", 1, 2, 128, 128, 64, "fp32", "none"),
        Workload("block_local_hiera", 128, 1, 3136, 3136, 96, "bf16", "block", 64),
        Workload("block_pooled_hiera", 128, 2, 784, 3136, 96, "bf16", "block", 64),
        Workload("global_vision", 128, 4, 196, 196, 96, "bf16", "none"),
        Workload("causal_lm", 1, 20, 8192, 8192, 128, "bf16", "causal"),
        Workload("sliding_pseudo_head", 1, 80, 4096, 4096, 128, "bf16", "sliding", 1024),
        Workload("iha_joint", 1, 20, 32768, 32768, 128, "bf16", "sliding", 1024, 4),
    )
}

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def make_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str = "bf16",
                seed: int = 0):
    """Return CPU tensors (q, k, v, do) drawn as the module docstring states."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((B, H, Nq, d), dtype=torch.float32, generator=g)
    k = torch.randn((B, H, Nk, d), dtype=torch.float32, generator=g)
    v = torch.randn((B, H, Nk, d), dtype=torch.float32, generator=g)
    do = torch.randn((B, H, Nq, d), dtype=torch.float32, generator=g)
    tdt = TORCH_DTYPES[dtype]
    if tdt is not torch.float32:
        q, k, v, do = (t.to(tdt) for t in (q, k, v, do))
    return q, k, v, do


def make_device_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str = "bf16",
                       seed: int = 0, device: str = "cuda"):
    """(q, k, v, do) drawn on the device, N(0, 1) in the requested type, from
    one generator of that device seeded with ``seed``, in that order: for
    tensors of several GB that the host would take minutes to draw.  The
    checks compare slices copied back to the host."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = TORCH_DTYPES[dtype]
    shapes = ((B, H, Nq, d), (B, H, Nk, d), (B, H, Nk, d), (B, H, Nq, d))
    return tuple(torch.randn(s, dtype=tdt, device=device, generator=g) for s in shapes)


def workload_inputs(w: Workload, seed: int = 0):
    return make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, seed)


def make_premix_inputs(B: int, N: int, H: int, P: int, d: int, dtype: str = "bf16",
                       seed: int = 0):
    """CPU tensors (x, w, dout) of an IHA premix: x [B, N, H, d] ~ N(0, 1),
    w [H, P, H] ~ N(0, 1/H) (so that each pseudo-head output has unit
    variance), dout [B, H, N, P, d] ~ N(0, 1); one generator seeded with
    ``seed``, drawn in that order in fp32, then rounded to ``dtype``."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((B, N, H, d), dtype=torch.float32, generator=g)
    w = torch.randn((H, P, H), dtype=torch.float32, generator=g) / math.sqrt(H)
    dout = torch.randn((B, H, N, P, d), dtype=torch.float32, generator=g)
    tdt = TORCH_DTYPES[dtype]
    return x.to(tdt), w.to(tdt), dout.to(tdt)
