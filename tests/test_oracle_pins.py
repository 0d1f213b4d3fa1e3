"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against scalar brute force, torch's own float64
``scaled_dot_product_attention`` (+ autograd), central finite differences,
a hand-derived worked example, closed forms, or invariants that the
mathematics of softmax attention fixes.  ``test_oracle_mutants.py`` shows
that planted mistakes in the oracle fail these pins.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import MASKS, oracle_bwd, oracle_fwd, visible
from oracle.brute import brute_fwd

RNG = np.random.default_rng(1234)

MASK_WINDOWS = [("none", 0), ("causal", 0), ("sliding", 3), ("block", 4)]


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- visibility

def _block_wq(window, nq, nk):
    """Query rows per block window (None: the shape has no block layout)."""
    if nk % window or nq % (nk // window):
        return None
    return nq // (nk // window)


@pytest.mark.parametrize("mask,window", MASK_WINDOWS + [("sliding", 1), ("block", 1), ("sliding", 40)])
@pytest.mark.parametrize("nq,nk", [(8, 8), (12, 12), (5, 9), (9, 5), (6, 12), (3, 12), (4, 8)])
def test_visibility_brute(mask, window, nq, nk):
    wq = _block_wq(window, nq, nk) if mask == "block" else 0
    if wq is None:
        pytest.skip("block mode needs Nk divisible by the block and Nq by the window count")
    from oracle.brute import sees
    vis = visible(mask, window, nq, nk)
    for i in range(nq):
        for j in range(nk):
            assert vis[i, j] == sees(mask, window, i, j, wq)


def test_block_rejects_shapes_without_windows():
    for nq, nk, w in ((8, 8, 3), (5, 8, 4), (7, 12, 4)):
        with pytest.raises(ValueError):
            visible("block", w, nq, nk)


def test_pooled_block_visibility_by_hand():
    """Nk = 8 keys in windows of 4 (two windows), Nq = 4 pooled query rows:
    rows 0, 1 belong to window 0 (keys 0..3), rows 2, 3 to window 1 (4..7)."""
    want = np.array([[1, 1, 1, 1, 0, 0, 0, 0],
                     [1, 1, 1, 1, 0, 0, 0, 0],
                     [0, 0, 0, 0, 1, 1, 1, 1],
                     [0, 0, 0, 0, 1, 1, 1, 1]], dtype=bool)
    assert (visible("block", 4, 4, 8) == want).all()


def test_visibility_special_cases():
    n = 16
    # sliding with W >= N is causal; block with w = N is no mask
    assert (visible("sliding", n, n, n) == visible("causal", 0, n, n)).all()
    assert (visible("sliding", 3 * n, n, n) == visible("causal", 0, n, n)).all()
    assert visible("block", n, n, n).all()
    # W = 1 and w = 1 keep only the diagonal
    eye = np.eye(n, dtype=bool)
    assert (visible("sliding", 1, n, n) == eye).all()
    assert (visible("block", 1, n, n) == eye).all()


def test_sliding_window_counts_match_wsl_table():
    """IHA-CUDA "FLOP Matching": window size W = WSL + 1.  With the table's
    first row (N = 8192, WSL = 1023) every row past the warm-up sees exactly
    WSL + 1 keys, and row i < WSL sees i + 1."""
    rows = _read_golden_table("iha_flop_matching.txt")
    n, wsl = rows[0]["N"], rows[0]["tile_matched_WSL"]
    assert (n, wsl) == (8192, 1023)
    probe = np.array([0, 1, 500, 1022, 1023, 1024, 4000, 8191])
    counts = visible("sliding", wsl + 1, n, n, rows=probe).sum(axis=1)
    expect = np.minimum(probe + 1, wsl + 1)
    assert (counts == expect).all()
    # the formula column of the same table: WSL = N / (2P) - 1 with P = 4
    for r in rows:
        assert r["formula_WSL"] == r["N"] // (2 * 4) - 1


def _read_golden_table(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    rows, header = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        cells = line.split()
        if header is None:
            header = cells
            continue
        rows.append({h: int(c) for h, c in zip(header, cells)})
    return rows


# ------------------------------------------------------- brute force (forward)

@pytest.mark.parametrize("mask,window", MASK_WINDOWS + [("sliding", 1)])
@pytest.mark.parametrize("nq,nk,d", [(8, 8, 4), (6, 9, 3), (9, 6, 5)])
def test_forward_vs_brute_force(mask, window, nq, nk, d):
    wq = 0
    if mask == "block":
        # equal windows, then pooled queries: 4 query rows over 8 keys
        nq, nk = {8: (8, 8), 6: (4, 8), 9: (2, 8)}[nq]
        wq = nq // (nk // window)
    B, H = 2, 2
    q, k, v = rand(B, H, nq, d), rand(B, H, nk, d), rand(B, H, nk, d)
    scale = 0.7
    o, lse = oracle_fwd(q, k, v, scale, mask, window)
    ob, lb = brute_fwd(q.tolist(), k.tolist(), v.tolist(), scale, mask, window, wq)
    ob, lb = np.array(ob), np.array(lb)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(lse[fin] - lb[fin])) < 1e-12
    assert np.max(np.abs(o - ob)) < 1e-12


# ------------------------------------------- library routine (fwd + autograd)

def _torch_sdpa(q, k, v, do, scale, mask, window):
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    vis = torch.tensor(visible(mask, window, q.shape[2], k.shape[2]))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=vis, scale=scale)
    (o * torch.tensor(do)).sum().backward()
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("mask,window", MASK_WINDOWS)
@pytest.mark.parametrize("n,d", [(16, 8), (24, 16)])
def test_against_torch_sdpa_fp64(mask, window, n, d):
    B, H = 2, 3
    q, k, v, do = (rand(B, H, n, d) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    o, _ = oracle_fwd(q, k, v, scale, mask, window)
    dq, dk, dv = oracle_bwd(q, k, v, do, scale, mask, window)
    to, tdq, tdk, tdv = _torch_sdpa(q, k, v, do, scale, mask, window)
    for a, b in ((o, to), (dq, tdq), (dk, tdk), (dv, tdv)):
        assert np.max(np.abs(a - b)) < 1e-10


def test_causal_matches_torch_is_causal():
    q, k, v = rand(1, 2, 12, 8), rand(1, 2, 12, 8), rand(1, 2, 12, 8)
    ref = F.scaled_dot_product_attention(*(torch.tensor(x) for x in (q, k, v)),
                                         is_causal=True, scale=0.3).numpy()
    o, _ = oracle_fwd(q, k, v, 0.3, "causal")
    assert np.max(np.abs(o - ref)) < 1e-12


# ------------------------------------------- central finite differences

@pytest.mark.parametrize("mask,window", MASK_WINDOWS + [("sliding", 2)])
def test_backward_finite_differences(mask, window):
    nq = nk = 8 if mask == "block" else 7
    if mask == "sliding" or mask == "causal":
        nq, nk = 7, 6          # also exercises Nq != Nk (top-left alignment)
    d = 3
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.standard_normal((1, 1, n, d)) for n in (nq, nk, nk, nq))
    scale = 0.9
    dq, dk, dv = oracle_bwd(q, k, v, do, scale, mask, window)

    def loss(q_, k_, v_):
        o, _ = oracle_fwd(q_, k_, v_, scale, mask, window)
        return float(np.sum(o * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd[idx] = (loss(**{f"{n}_": a for n, a in args_p.items()})
                       - loss(**{f"{n}_": a for n, a in args_m.items()})) / (2 * h)
        err = np.max(np.abs(fd - g)) / max(1.0, np.max(np.abs(g)))
        assert err < 1e-6, (name, err)


# ------------------------------------------- hand-derived worked example

def test_two_key_worked_example():
    """tests/golden/two_key_example.txt, derived by hand from the definition."""
    vals = {}
    import os
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "two_key_example.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            key, rest = line.split("=", 1)
            vals[key.strip()] = [eval(t, {"ln": math.log}) for t in rest.split()]
    q = np.array(vals["q"]).reshape(1, 1, 1, 2)
    k = np.array(vals["k"]).reshape(1, 1, 2, 2)
    v = np.array(vals["v"]).reshape(1, 1, 2, 2)
    do = np.array(vals["dO"]).reshape(1, 1, 1, 2)
    o, lse = oracle_fwd(q, k, v, vals["scale"][0], "none")
    dq, dk, dv = oracle_bwd(q, k, v, do, vals["scale"][0], "none")
    assert np.allclose(o.ravel(), vals["O"], atol=1e-14)
    assert np.allclose(lse.ravel(), vals["lse"], atol=1e-14)
    assert np.allclose(dq.ravel(), vals["dQ"], atol=1e-14)
    assert np.allclose(dk.ravel(), vals["dK"], atol=1e-14)
    assert np.allclose(dv.ravel(), vals["dV"], atol=1e-14)


# ------------------------------------------- closed forms

@pytest.mark.parametrize("mask,window", MASK_WINDOWS)
def test_rows_sum_to_one(mask, window):
    n, d = 16, 5
    q, k = rand(2, 2, n, d), rand(2, 2, n, d)
    o, _ = oracle_fwd(q, k, np.ones((2, 2, n, d)), 1.3, mask, window)
    assert np.max(np.abs(o - 1.0)) < 1e-13


@pytest.mark.parametrize("mask,window", MASK_WINDOWS)
def test_identical_keys_give_mean_of_visible_values(mask, window):
    n, d, scale = 16, 6, 0.4
    q, v = rand(1, 2, n, d), rand(1, 2, n, d)
    kvec = rand(d)
    k = np.broadcast_to(kvec, (1, 2, n, d)).copy()
    o, lse = oracle_fwd(q, k, v, scale, mask, window)
    vis = visible(mask, window, n, n)
    cnt = vis.sum(axis=1)
    mean_v = (vis[None, None].astype(float) @ v) / cnt[None, None, :, None]
    assert np.max(np.abs(o - mean_v)) < 1e-13
    assert np.max(np.abs(lse - (scale * q @ kvec + np.log(cnt)))) < 1e-12
    dq, _, _ = oracle_bwd(q, k, v, rand(1, 2, n, d), scale, mask, window)
    assert np.max(np.abs(dq)) < 1e-13


@pytest.mark.parametrize("mask,window", [("sliding", 1), ("block", 1)])
def test_single_visible_key_returns_its_value(mask, window):
    n, d, scale = 10, 4, 0.8
    q, k, v = rand(2, 1, n, d), rand(2, 1, n, d), rand(2, 1, n, d)
    o, lse = oracle_fwd(q, k, v, scale, mask, window)
    assert np.max(np.abs(o - v)) < 1e-14
    assert np.max(np.abs(lse - scale * np.sum(q * k, axis=-1))) < 1e-13


def test_single_key_sequence_and_causal_first_row():
    q, k, v = rand(1, 1, 5, 3), rand(1, 1, 1, 3), rand(1, 1, 1, 3)
    o, lse = oracle_fwd(q, k, v, 0.5, "none")
    assert np.max(np.abs(o - v)) < 1e-14
    assert np.max(np.abs(lse[0, 0] - 0.5 * q[0, 0] @ k[0, 0, 0])) < 1e-14
    q, k, v = rand(1, 1, 6, 3), rand(1, 1, 6, 3), rand(1, 1, 6, 3)
    o, lse = oracle_fwd(q, k, v, 0.5, "causal")
    assert np.max(np.abs(o[0, 0, 0] - v[0, 0, 0])) < 1e-14
    assert abs(lse[0, 0, 0] - 0.5 * q[0, 0, 0] @ k[0, 0, 0]) < 1e-14


@pytest.mark.parametrize("mask,window", MASK_WINDOWS)
def test_zero_scale_is_mean_of_visible(mask, window):
    n, d = 12, 3
    q, k, v = rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d)
    o, lse = oracle_fwd(q, k, v, 0.0, mask, window)
    vis = visible(mask, window, n, n).astype(float)
    cnt = vis.sum(axis=1)
    assert np.max(np.abs(o[0, 0] - (vis @ v[0, 0]) / cnt[:, None])) < 1e-14
    assert np.max(np.abs(lse[0, 0] - np.log(cnt))) < 1e-14


def test_reducing_special_cases():
    n, d = 12, 4
    q, k, v, do = (rand(1, 2, n, d) for _ in range(4))
    for (ma, wa), (mb, wb) in ((("sliding", n), ("causal", 0)),
                               (("sliding", 5 * n), ("causal", 0)),
                               (("block", n), ("none", 0))):
        oa, la = oracle_fwd(q, k, v, 0.6, ma, wa)
        ob, lb = oracle_fwd(q, k, v, 0.6, mb, wb)
        assert np.max(np.abs(oa - ob)) == 0 and np.max(np.abs(la - lb)) == 0
        ga = oracle_bwd(q, k, v, do, 0.6, ma, wa)
        gb = oracle_bwd(q, k, v, do, 0.6, mb, wb)
        for x, y in zip(ga, gb):
            assert np.max(np.abs(x - y)) == 0


# ------------------------------------------- invariants

def test_block_local_equals_dense_on_reshaped_windows():
    """hiera-optim mask_unit.py: windows are independent batches of a dense
    SDPA.  Block-local over N = nw * w equals mask none over (B*nw, H, w, d)."""
    B, H, nw, w, d = 2, 2, 3, 5, 4
    q, k, v, do = (rand(B, H, nw * w, d) for _ in range(4))

    def to_windows(x):
        return x.reshape(B, H, nw, w, d).transpose(0, 2, 1, 3, 4).reshape(B * nw, H, w, d)

    o, lse = oracle_fwd(q, k, v, 0.5, "block", w)
    ow, lw = oracle_fwd(to_windows(q), to_windows(k), to_windows(v), 0.5, "none")
    assert np.max(np.abs(to_windows(o) - ow)) < 1e-14
    assert np.max(np.abs(lse.reshape(B, H, nw, w).transpose(0, 2, 1, 3).reshape(B * nw, H, w) - lw)) < 1e-14
    g = oracle_bwd(q, k, v, do, 0.5, "block", w)
    gw = oracle_bwd(to_windows(q), to_windows(k), to_windows(v), to_windows(do), 0.5, "none")
    for x, y in zip(g, gw):
        assert np.max(np.abs(to_windows(x) - y)) < 1e-13


@pytest.mark.parametrize("nw,w,wq", [(3, 8, 2), (2, 4, 1), (4, 6, 3)])
def test_pooled_block_equals_dense_on_reshaped_windows(nw, w, wq):
    """hiera-optim MaskUnitAttentionFast with q_stride = w / wq: after the
    query pooling each window is an independent dense SDPA of wq queries over
    w keys.  Block-local with Nq = nw * wq, Nk = nw * w equals torch's float64
    SDPA (and its autograd) run per window with windows folded into the batch."""
    B, H, d, scale = 2, 2, 5, 0.45
    q, do = rand(B, H, nw * wq, d), rand(B, H, nw * wq, d)
    k, v = rand(B, H, nw * w, d), rand(B, H, nw * w, d)

    def to_windows(x, t):
        return x.reshape(B, H, nw, t, d).transpose(0, 2, 1, 3, 4).reshape(B * nw, H, t, d)

    o, lse = oracle_fwd(q, k, v, scale, "block", w)
    dq, dk, dv = oracle_bwd(q, k, v, do, scale, "block", w)
    qt, kt, vt = (torch.tensor(to_windows(x, t), requires_grad=True)
                  for x, t in ((q, wq), (k, w), (v, w)))
    ot = F.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    (ot * torch.tensor(to_windows(do, wq))).sum().backward()
    assert np.max(np.abs(to_windows(o, wq) - ot.detach().numpy())) < 1e-12
    lse_t = torch.logsumexp(scale * (qt @ kt.transpose(-1, -2)), dim=-1).detach().numpy()
    assert np.max(np.abs(lse.reshape(B, H, nw, wq).transpose(0, 2, 1, 3).reshape(B * nw, H, wq)
                         - lse_t)) < 1e-12
    for x, t, g in ((dq, wq, qt.grad), (dk, w, kt.grad), (dv, w, vt.grad)):
        assert np.max(np.abs(to_windows(x, t) - g.numpy())) < 1e-11


def test_pooled_block_backward_finite_differences():
    """Pooled-query block mask (Nq = 4, Nk = 8, window 4): gradients of
    sum(O * dO) against central differences."""
    rng = np.random.default_rng(11)
    q, do = rng.standard_normal((1, 1, 4, 3)), rng.standard_normal((1, 1, 4, 3))
    k, v = rng.standard_normal((1, 1, 8, 3)), rng.standard_normal((1, 1, 8, 3))
    grads = oracle_bwd(q, k, v, do, 0.8, "block", 4)
    h = 1e-6
    for which, g in enumerate(grads):
        args = [q, k, v]
        fd = np.zeros_like(args[which])
        for idx in np.ndindex(fd.shape):
            ap, am = [a.copy() for a in args], [a.copy() for a in args]
            ap[which][idx] += h
            am[which][idx] -= h
            fp = np.sum(oracle_fwd(*ap, 0.8, "block", 4)[0] * do)
            fm = np.sum(oracle_fwd(*am, 0.8, "block", 4)[0] * do)
            fd[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(fd - g)) < 1e-7


def test_key_value_permutation_invariance():
    n, d = 14, 5
    q, k, v, do = rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d), rand(1, 1, n, d)
    perm = RNG.permutation(n)
    o, lse = oracle_fwd(q, k, v, 0.7, "none")
    op, lp = oracle_fwd(q, k[:, :, perm], v[:, :, perm], 0.7, "none")
    assert np.max(np.abs(o - op)) < 1e-13 and np.max(np.abs(lse - lp)) < 1e-13
    dq, dk, dv = oracle_bwd(q, k, v, do, 0.7, "none")
    dqp, dkp, dvp = oracle_bwd(q, k[:, :, perm], v[:, :, perm], do, 0.7, "none")
    assert np.max(np.abs(dq - dqp)) < 1e-13
    assert np.max(np.abs(dk[:, :, perm] - dkp)) < 1e-13
    assert np.max(np.abs(dv[:, :, perm] - dvp)) < 1e-13


@pytest.mark.parametrize("mask,window", MASK_WINDOWS)
def test_key_offset_invariance(mask, window):
    n, d, scale = 16, 4, 0.8
    q, k, v = rand(1, 2, n, d), rand(1, 2, n, d), rand(1, 2, n, d)
    c = rand(d) * 3
    o, lse = oracle_fwd(q, k, v, scale, mask, window)
    o2, lse2 = oracle_fwd(q, k + c, v, scale, mask, window)
    assert np.max(np.abs(o - o2)) < 1e-12
    assert np.max(np.abs(lse2 - lse - scale * q @ c)) < 1e-12


def test_batch_head_permutation_equivariance():
    B, H, n, d = 3, 4, 10, 4
    q, k, v, do = (rand(B, H, n, d) for _ in range(4))
    pb, ph = RNG.permutation(B), RNG.permutation(H)

    def P(x):
        return x[pb][:, ph]

    o, lse = oracle_fwd(q, k, v, 0.5, "causal")
    op, lp = oracle_fwd(P(q), P(k), P(v), 0.5, "causal")
    assert np.array_equal(P(o), op) and np.array_equal(P(lse), lp)
    g = oracle_bwd(q, k, v, do, 0.5, "causal")
    gp = oracle_bwd(P(q), P(k), P(v), P(do), 0.5, "causal")
    for x, y in zip(g, gp):
        assert np.array_equal(P(x), y)


def test_value_scaling_and_gradient_linearity():
    n, d = 12, 4
    q, k, v, do, do2 = (rand(1, 1, n, d) for _ in range(5))
    o, _ = oracle_fwd(q, k, v, 0.5, "sliding", 4)
    o3, _ = oracle_fwd(q, k, 3.0 * v, 0.5, "sliding", 4)
    assert np.max(np.abs(3.0 * o - o3)) < 1e-13
    g1 = oracle_bwd(q, k, v, do, 0.5, "sliding", 4)
    g2 = oracle_bwd(q, k, v, do2, 0.5, "sliding", 4)
    g12 = oracle_bwd(q, k, v, 2.0 * do - do2, 0.5, "sliding", 4)
    for a, b, c in zip(g1, g2, g12):
        assert np.max(np.abs(2.0 * a - b - c)) < 1e-12


@pytest.mark.parametrize("mask,window", MASK_WINDOWS)
def test_gradient_sums(mask, window):
    """Rows of dS sum to zero (so sum_j dK_j = 0) and rows of P sum to one
    (so sum_j dV_j = sum_i dO_i), per (b, h) -- per window for block-local."""
    n, d = 16, 5
    q, k, v, do = (rand(2, 2, n, d) for _ in range(4))
    dq, dk, dv = oracle_bwd(q, k, v, do, 0.6, mask, window)
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12
    assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) < 1e-12
    if mask == "block":
        w = window
        assert np.max(np.abs(dk.reshape(2, 2, n // w, w, d).sum(axis=3))) < 1e-12
        assert np.max(np.abs(dv.reshape(2, 2, n // w, w, d).sum(axis=3)
                             - do.reshape(2, 2, n // w, w, d).sum(axis=3))) < 1e-12


def test_rows_without_visible_keys():
    """Sliding window with Nq > Nk + W - 1: the last rows see no key.  They get
    O = 0, lse = -inf, dQ = 0, and leave every other result unchanged."""
    nq, nk, W, d = 12, 6, 3, 4
    q, k, v, do = rand(1, 1, nq, d), rand(1, 1, nk, d), rand(1, 1, nk, d), rand(1, 1, nq, d)
    o, lse = oracle_fwd(q, k, v, 0.5, "sliding", W)
    dq, dk, dv = oracle_bwd(q, k, v, do, 0.5, "sliding", W)
    empty = np.arange(nq) >= nk + W - 1
    assert empty.sum() == 4
    assert np.all(o[0, 0, empty] == 0) and np.all(np.isneginf(lse[0, 0, empty]))
    assert np.all(dq[0, 0, empty] == 0)
    keep = ~empty
    o2, lse2 = oracle_fwd(q[:, :, keep], k, v, 0.5, "sliding", W)
    dq2, dk2, dv2 = oracle_bwd(q[:, :, keep], k, v, do[:, :, keep], 0.5, "sliding", W)
    assert np.max(np.abs(o2 - o[:, :, keep])) == 0
    assert np.max(np.abs(dk2 - dk)) < 1e-14 and np.max(np.abs(dv2 - dv)) < 1e-14


def test_widening_is_exact_for_bf16_inputs():
    """The oracle widens the very bf16 values the GPU receives: bf16 -> fp64
    is exact, so the oracle's inputs equal the device inputs bit for bit."""
    from head_attention_attn_amd.inputs import make_inputs
    q, k, v, do = make_inputs(1, 1, 8, 8, 64, "bf16", seed=0)
    assert torch.equal(torch.tensor(q.double().numpy()).to(torch.bfloat16), q)
