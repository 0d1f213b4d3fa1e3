"""Pins of the fp64 premix oracle (oracle/premix.py) against things other
than itself: a worked example done by hand (tests/golden/premix_example.txt),
scalar brute force with exactly rounded sums, the adjoint identities of a
bilinear map, finite differences, and special cases with known answers.
Planted mistakes in the oracle's source must fail them."""
import os

import numpy as np
import pytest

from oracle.brute import brute_premix, brute_premix_bwd
from oracle.premix import premix_bwd, premix_fwd, pseudo_tokens

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(77)
SRC = open(os.path.join(HERE, "..", "oracle", "premix.py")).read()


def golden():
    vals = {}
    for line in open(os.path.join(HERE, "golden", "premix_example.txt")):
        if line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        vals[k.strip()] = np.array([float(t) for t in v.split()])
    return vals


def test_worked_example(fwd=premix_fwd, bwd=premix_bwd):
    g = golden()
    x = g["x"].reshape(1, 1, 2, 2)
    w = g["w"].reshape(2, 2, 2)
    out = fwd(x, w)
    assert out.shape == (1, 2, 1, 2, 2)
    assert np.array_equal(out.reshape(-1), g["out"])
    dx, dw = bwd(x, w, g["dout"].reshape(1, 2, 1, 2, 2))
    assert np.array_equal(dx.reshape(-1), g["dx"])
    assert np.array_equal(dw.reshape(-1), g["dw"])


@pytest.mark.parametrize("B,N,H,P,d", [(1, 2, 3, 2, 2), (2, 3, 2, 4, 3), (1, 1, 4, 1, 5)])
def test_against_brute_force(B, N, H, P, d):
    x, w = RNG.standard_normal((B, N, H, d)), RNG.standard_normal((H, P, H))
    dout = RNG.standard_normal((B, H, N, P, d))
    out = premix_fwd(x, w)
    assert np.max(np.abs(out - np.array(brute_premix(x.tolist(), w.tolist())))) < 1e-13
    dx, dw = premix_bwd(x, w, dout)
    bdx, bdw = brute_premix_bwd(x.tolist(), w.tolist(), dout.tolist())
    assert np.max(np.abs(dx - np.array(bdx))) < 1e-13
    assert np.max(np.abs(dw - np.array(bdw))) < 1e-13


def test_adjoint_identities():
    """L(x, w, y) = <premix(x, w), y> is bilinear in (x, w): L = <x, dX(y)>
    and L = <w, dW(x, y)>."""
    B, N, H, P, d = 2, 5, 3, 4, 6
    x, w = RNG.standard_normal((B, N, H, d)), RNG.standard_normal((H, P, H))
    y = RNG.standard_normal((B, H, N, P, d))
    L = float(np.sum(premix_fwd(x, w) * y))
    dx, dw = premix_bwd(x, w, y)
    assert abs(L - float(np.sum(x * dx))) < 1e-10
    assert abs(L - float(np.sum(w * dw))) < 1e-10


def test_finite_differences():
    B, N, H, P, d = 1, 2, 2, 3, 2
    x, w = RNG.standard_normal((B, N, H, d)), RNG.standard_normal((H, P, H))
    y = RNG.standard_normal((B, H, N, P, d))
    dx, dw = premix_bwd(x, w, y)
    h = 1e-6
    for arr, grad, which in ((x, dx, 0), (w, dw, 1)):
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = (ap, w) if which == 0 else (x, ap)
            args_m = (am, w) if which == 0 else (x, am)
            fd = (np.sum(premix_fwd(*args_p) * y) - np.sum(premix_fwd(*args_m) * y)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7


def test_special_cases():
    B, N, H, d = 2, 3, 4, 5
    x = RNG.standard_normal((B, N, H, d))
    # P = 1 with W = I: each head's pseudo-tokens are that head's tokens
    out = premix_fwd(x, np.eye(H)[:, None, :])
    assert np.array_equal(out[:, :, :, 0, :], x.transpose(0, 2, 1, 3))
    # W[h, p, s] = [s == (h + p) mod H]: pseudo-head p of head h copies head h + p
    P = 3
    w = np.zeros((H, P, H))
    for h in range(H):
        for p in range(P):
            w[h, p, (h + p) % H] = 1.0
    out = premix_fwd(x, w)
    for h in range(H):
        for p in range(P):
            assert np.array_equal(out[:, h, :, p], x[:, :, (h + p) % H])
    # pseudo-token order: t = n * P + p
    seq = pseudo_tokens(out)
    assert np.array_equal(seq[:, 1, 2 * P + 1], x[:, 2, (1 + 1) % H])


MUTANTS = {
    "w_transposed": ('np.einsum("hps,bnsc->bhnpc", w, x)', 'np.einsum("sph,bnsc->bhnpc", w, x)'),
    "p_and_n_swapped": ('np.einsum("hps,bnsc->bhnpc", w, x)', 'np.einsum("hps,bnsc->bhpnc", w, x)'),
    "dx_untransposed": ('np.einsum("hps,bhnpc->bnsc", w, dout)', 'np.einsum("shp,bhnpc->bnsc", w, dout)'),
    "dw_wrong_operand": ('np.einsum("bhnpc,bnsc->hps", dout, x)',
                         'np.einsum("bhnpc,bnsc->hps", dout, x * x)'),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1
    ns = {"__name__": "premix_mutant"}
    exec(compile(SRC.replace(old, new), "premix_mutant", "exec"), ns)
    failed = False
    try:
        test_worked_example(ns["premix_fwd"], ns["premix_bwd"])
    except (AssertionError, ValueError):
        failed = True
    if not failed:  # the hand example may be blind to it: brute force at random shapes
        B, N, H, P, d = 1, 2, 3, 2, 2
        x, w = RNG.standard_normal((B, N, H, d)), RNG.standard_normal((H, P, H))
        y = RNG.standard_normal((B, H, N, P, d))
        try:
            o = ns["premix_fwd"](x, w)
            dx, dw = ns["premix_bwd"](x, w, y)
            failed = (o.shape != (B, H, N, P, d)
                      or np.max(np.abs(o - np.array(brute_premix(x.tolist(), w.tolist())))) > 1e-12)
            bdx, bdw = brute_premix_bwd(x.tolist(), w.tolist(), y.tolist())
            failed = failed or np.max(np.abs(dx - np.array(bdx))) > 1e-12 \
                or np.max(np.abs(dw - np.array(bdw))) > 1e-12
        except ValueError:
            failed = True
    assert failed, name
