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


def brute_premix(x, w):
    """IHA premix by scalar loops: x nested [B][N][H][d], w [H][P][H].
    Returns out [B][H][N][P][d] with out[b][h][n][p][c] = fsum over s of
    w[h][p][s] * x[b][n][s][c]."""
    B, N, H, d = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    P = len(w[0])
    return [[[[[math.fsum(w[h][p][s] * x[b][n][s][c] for s in range(H)) for c in range(d)]
               for p in range(P)] for n in range(N)] for h in range(H)] for b in range(B)]


def brute_premix_bwd(x, w, dout):
    """dX[b][n][s][c] = fsum over (h, p) of w[h][p][s] * dout[b][h][n][p][c];
    dW[h][p][s] = fsum over (b, n, c) of dout[b][h][n][p][c] * x[b][n][s][c]."""
    B, N, H, d = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    P = len(w[0])
    dx = [[[[math.fsum(w[h][p][s] * dout[b][h][n][p][c] for h in range(H) for p in range(P))
             for c in range(d)] for s in range(H)] for n in range(N)] for b in range(B)]
    dw = [[[math.fsum(dout[b][h][n][p][c] * x[b][n][s][c]
                      for b in range(B) for n in range(N) for c in range(d))
            for s in range(H)] for p in range(P)] for h in range(H)]
    return dx, dw
