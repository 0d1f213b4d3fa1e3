"""GPU parity of strided tensors (attn_fwd_strided / attn_bwd_strided).

The same seeded inputs are laid out two ways: contiguous [B, H, N, d] for the
oracle, and a strided arrangement for the HIP path -- Hiera's token order
(the qkv projection viewed as (B, T, nw, 3, H, D), token n = t * nw + w,
"hiera-optim 0.1.0" sdist, mask_unit.py, MaskUnitAttentionFast.forward) as
window-split [B, nw, H, T, D] views, or the sequence-major [B, N, H, d]
layout as transposed [B, H, N, d] views.  Results are compared with the
oracle element by element, and with the contiguous call bit for bit (the
kernels do the same arithmetic whatever the row addresses)."""
import numpy as np
import pytest
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd.inputs import make_inputs
from oracle import oracle_bwd, oracle_fwd

from _parity import compare, say, to64

pytestmark = pytest.mark.gpu


def token_order_buffer(B, T, nw, nslots, H, d, dtype):
    """A (B, T, nw, nslots, H, d) buffer: Hiera's token order (token
    n = t * nw + w) with ``nslots`` tensors interleaved per token."""
    return torch.zeros((B, T, nw, nslots, H, d), dtype=dtype, device="cuda")


def hiera_view(x4, buf, slot):
    """Write contiguous [B, H, nw*T, d] values (window-major tokens) into
    ``slot`` of a token-order buffer; return the [B, nw, H, T, d] view."""
    B, T, nw, _, H, d = buf.shape
    buf[:, :, :, slot] = x4.view(B, H, nw, T, d).permute(0, 3, 2, 1, 4).cuda()
    return buf[:, :, :, slot].permute(0, 2, 3, 1, 4)


def from_windows(x5):
    """[B, nw, H, T, d] view -> contiguous [B, H, nw*T, d] (window-major)."""
    B, nw, H, T, d = x5.shape
    return x5.permute(0, 2, 1, 3, 4).reshape(B, H, nw * T, d)


def oracle_case(q, k, v, do, scale, mask, window):
    ro, rl = oracle_fwd(to64(q), to64(k), to64(v), scale, mask, window)
    rg = oracle_bwd(to64(q), to64(k), to64(v), to64(do), scale, mask, window)
    return (ro, rl) + tuple(rg)


@pytest.mark.parametrize("nw,T,Tq,H,d", [
    (7, 64, 16, 2, 96),      # pooled (q_stride 4), single-tile kernels
    (5, 64, 64, 2, 64),      # unpooled 64-token mask units, single-tile kernels
    (3, 128, 32, 2, 96),     # 128-key windows: general kernels, interleaved windows
    (3, 128, 64, 1, 128),    # d = 128: dK/dV keeps dS for the dQ pass
])
def test_hiera_token_order(nw, T, Tq, H, d):
    """K, V read in place from one qkv buffer in Hiera's token order, Q and
    dO in their own (B, Tq, nw, H, d) buffers, dK and dV written into one
    interleaved dkv buffer, O and dQ in token order."""
    B = 2
    say(f"[strided hiera] B={B} nw={nw} T={T} Tq={Tq} H={H} d={d}")
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    q, k, v, do = make_inputs(B, H, nw * Tq, nw * T, d, "bf16", seed=20)
    qkv = token_order_buffer(B, T, nw, 3, H, d, torch.bfloat16)
    k5, v5 = hiera_view(k, qkv, 1), hiera_view(v, qkv, 2)
    if Tq == T:
        q5 = hiera_view(q, qkv, 0)
    else:  # pooled queries live in their own (B, Tq, nw, H, d) buffer
        q5 = hiera_view(q, token_order_buffer(B, Tq, nw, 1, H, d, torch.bfloat16), 0)
    do5 = hiera_view(do, token_order_buffer(B, Tq, nw, 1, H, d, torch.bfloat16), 0)
    dkv = torch.full((B, T, nw, 2, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    dk5 = dkv[:, :, :, 0].permute(0, 2, 3, 1, 4)
    dv5 = dkv[:, :, :, 1].permute(0, 2, 3, 1, 4)

    o5, lse = attn.fwd(q5, k5, v5, scale=scale)
    dq5, _, _ = attn.bwd(q5, k5, v5, o5, lse, do5, scale=scale, dk=dk5, dv=dv5)
    torch.cuda.synchronize()
    assert o5.shape == q5.shape and o5.stride()[1] == H * d      # token order, windows fastest
    ro, rl, rdq, rdk, rdv = oracle_case(q, k, v, do, scale, "block", T)
    rep = compare([("O", to64(from_windows(o5)), ro), ("lse", to64(lse), rl),
                   ("dQ", to64(from_windows(dq5)), rdq), ("dK", to64(from_windows(dk5)), rdk),
                   ("dV", to64(from_windows(dv5)), rdv)], "bf16", label=f"hiera T{T} Tq{Tq} d{d}")
    say(f"[strided hiera] {rep}")

    # the same inputs contiguous: bitwise the same results
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    oc, lc = attn.fwd(qc, kc, vc, mask="block", window=T, scale=scale)
    dqc, dkc, dvc = attn.bwd(qc, kc, vc, oc, lc, doc, mask="block", window=T, scale=scale)
    torch.cuda.synchronize()
    for a, b in ((from_windows(o5), oc), (lse, lc), (from_windows(dq5), dqc),
                 (from_windows(dk5), dkc), (from_windows(dv5), dvc)):
        assert torch.equal(a, b)


def seq_major(x4, pad=0):
    """[B, H, N, d] values as a view of a sequence-major (B, N, H, d + pad)
    buffer (rows of d + pad elements when padded)."""
    B, H, N, d = x4.shape
    buf = torch.zeros((B, N, H, d + pad), dtype=x4.dtype, device="cuda")
    buf[..., :d] = x4.permute(0, 2, 1, 3).cuda()
    return buf[..., :d].permute(0, 2, 1, 3)


@pytest.mark.parametrize("dtype,d,nq,nk,mask,window,pad", [
    ("bf16", 64, 200, 200, "causal", 0, 0),
    ("bf16", 96, 150, 77, "none", 0, 8),
    ("bf16", 128, 333, 333, "sliding", 70, 0),
    ("bf16", 128, 130, 130, "causal", 0, 16),
    ("fp32", 64, 100, 37, "causal", 0, 4),
    ("fp32", 128, 70, 70, "sliding", 9, 0),
])
def test_sequence_major_layout(dtype, d, nq, nk, mask, window, pad):
    """Every tensor, outputs included, as a [B, N, H, d] buffer viewed as
    [B, H, N, d] (rows padded by ``pad`` elements where given)."""
    B, H = 2, 3
    say(f"[strided seq-major] {dtype} d={d} {nq}x{nk} {mask} W={window} pad={pad}")
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    q, k, v, do = make_inputs(B, H, nq, nk, d, dtype, seed=21)
    qs, ks, vs, dos = (seq_major(t, pad) for t in (q, k, v, do))
    o = seq_major(torch.zeros_like(q), pad)
    dq, dk, dv = (seq_major(torch.zeros_like(t), pad) for t in (q, k, v))
    assert not qs.is_contiguous()
    o, lse = attn.fwd(qs, ks, vs, mask=mask, window=window, scale=scale, out=o)
    attn.bwd(qs, ks, vs, o, lse, dos, mask=mask, window=window, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ro, rl, rdq, rdk, rdv = oracle_case(q, k, v, do, scale, mask, window)
    rep = compare([("O", to64(o), ro), ("lse", to64(lse), rl), ("dQ", to64(dq), rdq),
                   ("dK", to64(dk), rdk), ("dV", to64(dv), rdv)], dtype,
                  label=f"seq-major {dtype} d{d} {mask}")
    say(f"[strided seq-major] {rep}")
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    oc, lc = attn.fwd(qc, kc, vc, mask=mask, window=window, scale=scale)
    dqc, dkc, dvc = attn.bwd(qc, kc, vc, oc, lc, doc, mask=mask, window=window, scale=scale)
    torch.cuda.synchronize()
    for a, b in ((o, oc), (lse, lc), (dq, dqc), (dk, dkc), (dv, dvc)):
        assert torch.equal(a, b)


def test_strided_outputs_leave_the_gaps_alone():
    """Padded sequence-major outputs: the pad elements between rows keep
    their canary value."""
    B, H, N, d, pad = 1, 2, 96, 64, 8
    q, k, v, do = make_inputs(B, H, N, N, d, "bf16", seed=22)
    qs, ks, vs, dos = (seq_major(t) for t in (q, k, v, do))
    obuf = torch.full((B, N, H, d + pad), 5.0, dtype=torch.bfloat16, device="cuda")
    o = obuf[..., :d].permute(0, 2, 1, 3)
    attn.fwd(qs, ks, vs, mask="causal", out=o)
    torch.cuda.synchronize()
    assert bool((obuf[..., d:] == 5.0).all())
