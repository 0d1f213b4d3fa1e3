"""Plain float64 attention: the definition, materialised, row-chunked only to
bound memory.  TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (cited by page title and section):

* IHA-CUDA README ("Interleaved Head Attention Kernels for Hopper GPUs"),
  "FLOP Matching": the sliding window has size W = WSL + 1, i.e. W counts the
  visible keys of a row including the diagonal.
* hiera-optim 0.1.0 sdist, ``hiera_optim/attention/mask_unit.py``
  (``MaskUnitAttentionFast.forward``): mask-unit attention splits the tokens
  into independent windows and runs a dense SDPA inside each window, with the
  default scale head_dim ** -0.5.  Windows here are contiguous runs of
  ``window`` tokens (the permute that makes them contiguous is the caller's).
* The problem statement of this library: softmax(Q K^T * scale + mask) V with
  mask modes none / causal / causal sliding window / block-local, the per-row
  logsumexp, and dQ, dK, dV from dO.

Readings where the pages are silent (each is listed in the design notes):

* lse is the natural-log logsumexp of the *scaled* scores.
* A row with no visible key has O = 0 and lse = -inf and contributes nothing
  to any gradient (dQ row = 0).
* Causal and sliding masks are top-left aligned on absolute indices
  (key j visible to query i iff j <= i [and j > i - W]), also when Nq != Nk.
* Block-local: query i and key j see each other iff they fall in the same
  window.  With Nq == Nk the windows are floor(i/w) == floor(j/w).  With
  pooled queries (hiera-optim ``MaskUnitAttentionFast.forward`` with
  ``q_stride > 1``: Q is max-pooled inside each window, so a window holds
  T keys but only T / q_stride queries, and SDPA runs per window on those),
  the Nk / w windows of w keys each hold Nq / (Nk / w) consecutive query rows.
"""
from __future__ import annotations

import numpy as np

MASKS = ("none", "causal", "sliding", "block")

_ROW_CHUNK = 512


def visible(mask: str, window: int, nq: int, nk: int, rows=None) -> np.ndarray:
    """Boolean visibility matrix vis[i, j] for query rows ``rows`` (default all).

    none    -> every key
    causal  -> j <= i
    sliding -> i - window < j <= i         (window >= 1 keys incl. the diagonal)
    block   -> same window: floor(i / wq) == floor(j / window) with
               nw = nk / window windows and wq = nq / nw query rows per
               window (wq = window when nq == nk)
    """
    i = np.arange(nq) if rows is None else np.asarray(rows)
    i = i[:, None]
    j = np.arange(nk)[None, :]
    if mask == "none":
        return np.ones((i.shape[0], nk), dtype=bool)
    if mask == "causal":
        return j <= i
    if mask == "sliding":
        if window < 1:
            raise ValueError("sliding window must be >= 1")
        return (j <= i) & (j > i - window)
    if mask == "block":
        if window < 1 or nk % window:
            raise ValueError("block length must be >= 1 and divide nk")
        nw = nk // window
        if nq % nw:
            raise ValueError("block mode needs nq divisible by the number of windows")
        return (i // (nq // nw)) == (j // window)
    raise ValueError(f"unknown mask {mask!r}")


def _probs(q2, k2, scale, vis):
    """Scores, masked, turned into probabilities and the row logsumexp.

    s_ij = scale * <q_i, k_j> where visible, -inf elsewhere;
    lse_i = m_i + ln sum_j exp(s_ij - m_i) with m_i = max_j s_ij;
    P_ij = exp(s_ij - lse_i).   Empty rows: P = 0, lse = -inf.
    """
    s = scale * (q2 @ k2.T)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe)                     # exp(-inf) = 0 on masked entries
    tot = e.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    p = np.where(empty, 0.0, e / np.where(empty, 1.0, tot))
    return p, lse[:, 0]


def _as64(x):
    x = np.asarray(x)
    if x.dtype != np.float64:
        x = x.astype(np.float64)
    return x


def oracle_fwd(q, k, v, scale: float, mask: str = "none", window: int = 0):
    """Forward attention.  q: [B,H,Nq,d], k, v: [B,H,Nk,d] (any float dtype,
    widened exactly to float64).  Returns O [B,H,Nq,d] and lse [B,H,Nq],
    both float64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, nq, d = q.shape
    nk = k.shape[2]
    scale = float(scale)
    o = np.zeros((B, H, nq, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, nq, _ROW_CHUNK):
                rows = np.arange(r0, min(nq, r0 + _ROW_CHUNK))
                vis = visible(mask, window, nq, nk, rows)
                p, l = _probs(q[b, h, rows], k[b, h], scale, vis)
                o[b, h, rows] = p @ v[b, h]
                lse[b, h, rows] = l
    return o, lse


def oracle_bwd(q, k, v, do, scale: float, mask: str = "none", window: int = 0):
    """Gradients of L = sum(O * dO) with respect to Q, K, V.

    Uses the softmax Jacobian directly: with dP = dO V^T,
    dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik); then dQ = scale * dS K,
    dK = scale * dS^T Q, dV = P^T dO.  P is recomputed here from Q and K; no
    forward output is taken from outside.  Returns float64 dq, dk, dv.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, nq, d = q.shape
    nk = k.shape[2]
    scale = float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros((B, H, nk, d), dtype=np.float64)
    dv = np.zeros((B, H, nk, v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, nq, _ROW_CHUNK):
                rows = np.arange(r0, min(nq, r0 + _ROW_CHUNK))
                vis = visible(mask, window, nq, nk, rows)
                p, _ = _probs(q[b, h, rows], k[b, h], scale, vis)
                dp = do[b, h, rows] @ v[b, h].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h, rows] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, rows])
                dv[b, h] += p.T @ do[b, h, rows]
    return dq, dk, dv
