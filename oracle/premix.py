"""Plain float64 IHA premix (pseudo-token construction) and its gradients.
TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "IHA-CUDA: Interleaved Head Attention Kernels for Hopper GPUs",
section "Pseudo-Token Mixing (Triton Premix Kernels)": before attention, Q, K
and V are each mixed across heads by a learned weight,

    Out[h, p] = sum_s W[h, p, s] * X[s],

a linear map from H source heads to H x P pseudo-heads applied independently
at every (batch, position, feature) coordinate; its backward is
dX = W^T dOut (the transpose of that map) and dW = sum over (b, n, feature)
of dOut * X^T.

Layouts (readings, also listed in the design notes):

* X   [B][N][H][d]     -- a projection output, position-major;
* W   [H][P][H]        -- W[h, p, s];
* Out [B][H][N][P][d]  -- per head h, the N * P pseudo-tokens in the order
  t = n * P + p.  Attention with a joint softmax across the P pseudo-heads
  ("IHA-CUDA", introduction and Kernel Design: a nested loop over query
  pseudo-tokens and key-value pairs) is then ordinary attention over that
  pseudo-token sequence; with a causal window of W = WSL + 1 pseudo-tokens
  and WSL = N / (2P) - 1 ("FLOP Matching") it visits N^2 / 2 (query, key)
  pairs per head, as causal attention over the N tokens does.

Each function is the definition written out with ``numpy.einsum`` (a library
contraction used as one step); nothing is blocked or reordered.
"""
from __future__ import annotations

import numpy as np


def premix_fwd(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Out[b, h, n, p, c] = sum_s W[h, p, s] * X[b, n, s, c]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return np.einsum("hps,bnsc->bhnpc", w, x)


def premix_bwd(x: np.ndarray, w: np.ndarray, dout: np.ndarray):
    """Gradients of L = <premix_fwd(x, w), dout>:
    dX[b, n, s, c] = sum_{h, p} W[h, p, s] * dOut[b, h, n, p, c]   (W^T dOut)
    dW[h, p, s]    = sum_{b, n, c} dOut[b, h, n, p, c] * X[b, n, s, c]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    dx = np.einsum("hps,bhnpc->bnsc", w, dout)
    dw = np.einsum("bhnpc,bnsc->hps", dout, x)
    return dx, dw


def pseudo_tokens(out: np.ndarray) -> np.ndarray:
    """[B][H][N][P][d] -> [B][H][N * P][d]: pseudo-token t = n * P + p."""
    B, H, N, P, d = out.shape
    return out.reshape(B, H, N * P, d)
