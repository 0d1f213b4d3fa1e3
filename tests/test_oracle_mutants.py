"""Planted mistakes in the oracle must fail its pins.

Each mutant is the oracle's own source with one plausible mistake edited in
(a dropped term, a wrong sign, an off-by-one in a mask, a wrong operand, a
wrong log base).  It is executed into a private namespace on the CPU; the
real oracle is untouched.  A mutant that passed every pin would mean the pins
could not tell that mistake from the right answer.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.brute import brute_fwd, sees

SRC = open(os.path.join(os.path.dirname(__file__), "..", "oracle", "attention.py")).read()

MUTANTS = {
    "dropped_softmax_jacobian_term": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "wrong_sign_jacobian": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                            "ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))"),
    "dq_missing_scale": ("dq[b, h, rows] = scale * (ds @ k[b, h])", "dq[b, h, rows] = (ds @ k[b, h])"),
    "dk_wrong_operand": ("dk[b, h] += scale * (ds.T @ q[b, h, rows])",
                         "dk[b, h] += scale * (ds.T @ do[b, h, rows])"),
    "dv_untransposed_probs": ("dv[b, h] += p.T @ do[b, h, rows]",
                              "dv[b, h] += (p.T @ do[b, h, rows])[::-1]"),
    "causal_strict": ("        return j <= i\n", "        return j < i\n"),
    "sliding_off_by_one": ("return (j <= i) & (j > i - window)", "return (j <= i) & (j >= i - window)"),
    "block_modulo": ("return (i // (nq // nw)) == (j // window)", "return (i % (nq // nw)) == (j % window)"),
    "block_query_window_unpooled": ("return (i // (nq // nw)) == (j // window)",
                                    "return (i // window) == (j // window)"),
    "lse_log2": ("m_safe + np.log(np.where(empty, 1.0, tot))", "m_safe + np.log2(np.where(empty, 1.0, tot))"),
    "scores_unscaled": ("s = scale * (q2 @ k2.T)", "s = (q2 @ k2.T)"),
    "transposed_scores": ("s = scale * (q2 @ k2.T)", "s = scale * (q2 @ k2.T)[:, ::-1]"),
}


def _load(mutation):
    old, new = mutation
    assert SRC.count(old) == 1, old
    ns = {"__name__": "oracle_mutant"}
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), ns)
    return ns


def _pins_pass(ns) -> bool:
    """The pins, compactly: brute force, torch fp64 SDPA + autograd, closed forms."""
    rng = np.random.default_rng(5)
    fwd, bwd, vis = ns["oracle_fwd"], ns["oracle_bwd"], ns["visible"]
    try:
        for mask, window, nq in (("none", 0, 8), ("causal", 0, 8), ("sliding", 3, 8), ("block", 4, 8),
                                 ("block", 4, 4)):
            n, d, scale = 8, 4, 0.7
            wq = nq // (n // window) if mask == "block" else 0
            q, do = (rng.standard_normal((1, 2, nq, d)) for _ in range(2))
            k, v = (rng.standard_normal((1, 2, n, d)) for _ in range(2))
            # brute force forward with an independent visibility rule
            o, lse = fwd(q, k, v, scale, mask, window)
            ob, lb = brute_fwd(q.tolist(), k.tolist(), v.tolist(), scale, mask, window, wq)
            if np.max(np.abs(o - np.array(ob))) > 1e-12 or np.max(np.abs(lse - np.array(lb))) > 1e-12:
                return False
            # library routine with autograd; its mask built by the brute-force rule
            m = torch.tensor([[sees(mask, window, i, j, wq) for j in range(n)] for i in range(nq)])
            qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
            ot = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
            (ot * torch.tensor(do)).sum().backward()
            g = bwd(q, k, v, do, scale, mask, window)
            for a, b in zip(g, (qt.grad, kt.grad, vt.grad)):
                if np.max(np.abs(a - b.numpy())) > 1e-10:
                    return False
            # closed form: V = 1 gives O = 1
            o1, _ = fwd(q, k, np.ones_like(v), scale, mask, window)
            if np.max(np.abs(o1 - 1)) > 1e-12:
                return False
    except Exception:
        return False
    return True


def test_unmutated_oracle_passes_compact_pins():
    assert _pins_pass(_load(("s = scale * (q2 @ k2.T)", "s = scale * (q2 @ k2.T)")))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert not _pins_pass(_load(MUTANTS[name])), f"mutant {name} passed every pin"
