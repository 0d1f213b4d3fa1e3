"""Scalar brute-force attention for tiny inputs.  TEST INFRASTRUCTURE ONLY.

Pure-Python loops over nested lists with ``math.fsum`` (exactly rounded
sums) and the visibility rule written as an explicit per-pair test, so that
it shares neither vectorisation nor masking code with ``attention``.  It is
here to pin the vectorised oracle; it is far too slow for anything but
B, H <= 2, N <= 16, d <= 8.

The forward follows the definition softmax(scale * q_i . k_j over the visible
j) weighted sum of v_j (hiera-optim ``MaskUnitAttentionFast.forward`` calls
SDPA with default scale head_dim ** -0.5; IHA-CUDA "FLOP Matching" gives the
window as W = WSL + 1 keys).
"""
from __future__ import annotations

import math


def sees(mask: str, window: int, i: int, j: int, window_q: int = 0) -> bool:
    """Is key j visible to query i.  block: query i lies in window
    i // window_q (window_q query rows per window; default ``window``) and key
    j in window j // window."""
    if mask == "none":
        return True
    if mask == "causal":
        return j <= i
    if mask == "sliding":
        return i - window < j <= i
    if mask == "block":
        return i // (window_q or window) == j // window
    raise ValueError(mask)


def brute_fwd(q, k, v, scale, mask="none", window=0, window_q=0):
    """q, k, v: nested lists [B][H][N][d] of floats.  Returns (o, lse) lists.
    ``window_q``: query rows per block window when queries are pooled."""
    B, H = len(q), len(q[0])
    o, lse = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(H):
            oh, lh = [], []
            Q, K, V = q[b][h], k[b][h], v[b][h]
            for i in range(len(Q)):
                js = [j for j in range(len(K)) if sees(mask, window, i, j, window_q)]
                if not js:
                    oh.append([0.0] * len(V[0]))
                    lh.append(-math.inf)
                    continue
                s = {j: scale * math.fsum(Q[i][c] * K[j][c] for c in range(len(Q[i]))) for j in js}
                mx = max(s.values())
                z = math.fsum(math.exp(s[j] - mx) for j in js)
                lh.append(mx + math.log(z))
                w = {j: math.exp(s[j] - mx) / z for j in js}
                oh.append([math.fsum(w[j] * V[j][c] for j in js) for c in range(len(V[0]))])
            ob.append(oh)
            lb.append(lh)
        o.append(ob)
        lse.append(lb)
    return o, lse
