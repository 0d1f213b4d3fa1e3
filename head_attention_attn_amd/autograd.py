"""torch.autograd bridge over the C ABI: the fused attention as a
differentiable op and as an ``nn.Module``.

The forward calls ``attn_fwd`` and saves O and the per-row logsumexp; the
backward calls ``attn_bwd`` with them and the incoming dO.  This is how the
pages put fused attention kernels under a model: "IHA-CUDA" (End-to-End
Training Benchmark) has its baseline attention layer call the forward and
backward kernels through a ``torch.autograd.Function`` wrapper, and
"hiera-optim 0.1.0" (sdist ``hiera_optim/attention/mask_unit.py``,
``MaskUnitAttentionFast``) is an ``nn.Module`` whose attention core takes
q, k, v of shape [batch, heads, tokens, head_dim] and returns O of that
shape.  Nothing here does arithmetic on the tensors: shapes are
checked, and every product and softmax runs in the library's kernels.
"""
from __future__ import annotations

import torch

from . import binding


class FusedAttentionFunction(torch.autograd.Function):
    """O = softmax(scale * Q K^T + mask) V, with dQ, dK, dV from ``attn_bwd``.

    Inputs: device tensors q [B, H, Nq, d], k and v [B, H, Nk, d] with any
    row strides (views of a projection output need no copy), or window-split
    [B, nw, H, T, d] views for the block mask (bf16, fp16 or fp32); the mask
    name, its window and the scale (None: d^-0.5).  Returns O shaped like q.
    ``keep_ds`` picks the backward workspace: large enough for the dQ pass to
    read dS kept by the dK/dV pass where that path applies
    (``attn_bwd_workspace_size_ds``), else the minimum."""

    @staticmethod
    def forward(ctx, q, k, v, mask="none", window=0, scale=None, keep_ds=True):
        o, lse = binding.fwd(q, k, v, mask=mask, window=window, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (mask, window, scale, keep_ds)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        mask, window, scale, keep_ds = ctx.cfg
        # dO in q's dtype; the kernels take any row strides, but a broadcast
        # (stride 0) or unaligned gradient is copied first
        do = do.to(q.dtype)
        if not binding.rows_usable(do):
            do = do.contiguous()
        dq, dk, dv = binding.bwd(q, k, v, o, lse, do, mask=mask, window=window, scale=scale,
                                 keep_ds=keep_ds)
        return dq, dk, dv, None, None, None, None


def fused_attention(q, k, v, mask: str = "none", window: int = 0, scale=None,
                    keep_ds: bool = True):
    """Differentiable fused attention (see ``FusedAttentionFunction``)."""
    return FusedAttentionFunction.apply(q, k, v, mask, window, scale, keep_ds)


class FusedAttention(torch.nn.Module):
    """The attention core of a transformer layer as a module: no parameters;
    ``forward(q, k, v)`` with q [B, H, Nq, d], k, v [B, H, Nk, d] returns O
    [B, H, Nq, d].  ``mask`` is "none", "causal", "sliding" (``window`` keys
    including the diagonal) or "block" (independent windows of ``window``
    keys, the mask-unit case; each window holds Nq / (Nk / window) query rows,
    fewer than ``window`` when queries are pooled); ``scale`` defaults to
    d^-0.5."""

    def __init__(self, mask: str = "none", window: int = 0, scale=None, keep_ds: bool = True):
        super().__init__()
        if mask not in binding.MASK_CODES:
            raise ValueError(f"unknown mask {mask!r}")
        self.mask, self.window, self.scale, self.keep_ds = mask, int(window), scale, keep_ds

    def forward(self, q, k, v):
        return fused_attention(q, k, v, self.mask, self.window, self.scale, self.keep_ds)

    def extra_repr(self) -> str:
        return f"mask={self.mask!r}, window={self.window}, scale={self.scale}"


class PremixFunction(torch.autograd.Function):
    """IHA pseudo-token construction out = premix(x, w) ("IHA-CUDA",
    Pseudo-Token Mixing) with its backward from ``attn_premix_bwd``: x
    [B, N, H, d], w [H, P, H] (x's dtype) -> [B, H, N, P, d]."""

    @staticmethod
    def forward(ctx, x, w):
        ctx.save_for_backward(x, w)
        return binding.premix(x, w)

    @staticmethod
    def backward(ctx, dout):
        x, w = ctx.saved_tensors
        dx, dw = binding.premix_bwd(x, w, dout.to(x.dtype).contiguous())
        return dx, dw.to(w.dtype)


def premix(x, w):
    """Differentiable IHA premix (see ``PremixFunction``)."""
    return PremixFunction.apply(x, w)


def iha_attention(xq, xk, xv, wq, wk, wv, window: int, scale=None):
    """Interleaved head attention: Q, K, V premixed into P pseudo-heads per
    head, then one causal sliding-window attention of ``window`` pseudo-tokens
    over each head's N * P pseudo-tokens (the joint softmax across
    pseudo-heads).  x* [B, N, H, d], w* [H, P, H]; returns O [B, H, N * P, d]
    (pseudo-token t = n * P + p)."""
    B, N, H, d = xq.shape
    P = wq.shape[1]
    q, k, v = (premix(x, w).view(B, H, N * P, d) for x, w in ((xq, wq), (xk, wk), (xv, wv)))
    return fused_attention(q, k, v, "sliding", window, scale)
