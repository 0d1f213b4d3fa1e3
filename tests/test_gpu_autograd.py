"""The autograd bridge (``head_attention_attn_amd.autograd``): gradients that
reach q, k, v through ``loss.backward()`` are the C ABI's dQ, dK, dV, checked
against the fp64 oracle on the same seeded inputs and loss, and the module
composes with ordinary torch ops (a projection before it, a reduction after)."""
import numpy as np
import pytest
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd.inputs import make_inputs
from oracle import oracle_bwd, oracle_fwd

from _parity import compare, say, to64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d,mask,window,n", [
    ("bf16", 128, "causal", 0, 200), ("bf16", 96, "block", 64, 192),
    ("bf16", 64, "sliding", 37, 150), ("fp32", 64, "none", 0, 77),
])
def test_autograd_gradients_match_oracle(dtype, d, mask, window, n):
    """L = <O, dO>: autograd's q.grad, k.grad, v.grad equal the oracle's dQ,
    dK, dV for that loss.  Short causal rows make the first keys' dV entries
    reach |5|, where rounding the bf16 output alone costs up to 2^-8 * |x|
    (0.02): the max-abs bound grows by 2^-8 * max|ref| (rel-L2 keeps 5e-3)."""
    say(f"[autograd] {dtype} d={d} {mask} W={window} N={n}")
    q, k, v, do = make_inputs(2, 2, n, n, d, dtype, seed=21)
    scale = float(torch.tensor(1.0 / np.sqrt(d), dtype=torch.float32))
    qd, kd, vd = (t.cuda().requires_grad_(True) for t in (q, k, v))
    o = attn.fused_attention(qd, kd, vd, mask=mask, window=window, scale=scale)
    loss = (o.float() * do.cuda().float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    ro, _ = oracle_fwd(to64(q), to64(k), to64(v), scale, mask, window)
    rdq, rdk, rdv = oracle_bwd(to64(q), to64(k), to64(v), to64(do), scale, mask, window)
    compare([("O", to64(o), ro), ("dQ", to64(qd.grad), rdq), ("dK", to64(kd.grad), rdk),
             ("dV", to64(vd.grad), rdv)], dtype, f"autograd {mask}",
            amax_rel=2.0 ** -8 if dtype == "bf16" else 0.0)


@pytest.mark.parametrize("copy", [True, False])
def test_module_inside_a_graph(copy):
    """x -> q, k, v by a linear map -> FusedAttention -> mean: the gradient of
    the linear map's weight matches the same graph with the oracle's attention
    gradient chained by hand (dW = sum over rows of x^T [dQ dK dV] for the
    per-head split used here).  ``copy``: q, k, v made contiguous first, or
    read in place as strided views of the projection output."""
    torch.manual_seed(0)
    B, H, N, d = 1, 2, 130, 64
    x = torch.randn(B, N, H * d)
    w = torch.randn(H * d, 3 * H * d) * (H * d) ** -0.5
    xd, wd = x.cuda(), w.cuda().requires_grad_(True)
    qkv = (xd @ wd).view(B, N, 3, H, d).permute(2, 0, 3, 1, 4)
    if copy:
        qkv = qkv.contiguous()
    layer = attn.FusedAttention(mask="causal")
    q, k, v = (qkv[i].contiguous() if copy else qkv[i] for i in range(3))
    assert copy or not q.is_contiguous()
    o = layer(q, k, v)
    o.mean().backward()
    torch.cuda.synchronize()
    # oracle: same graph in fp64 on the CPU, attention gradient from the oracle
    x64, w64 = x.double().numpy(), w.double().numpy()
    qkv64 = (x64 @ w64).reshape(B, N, 3, H, d).transpose(2, 0, 3, 1, 4)
    q64, k64, v64 = qkv64[0], qkv64[1], qkv64[2]
    do64 = np.full(q64.shape, 1.0 / q64.size)
    dq, dk, dv = oracle_bwd(q64, k64, v64, do64, d ** -0.5, "causal", 0)
    dqkv = np.stack([dq, dk, dv])                                  # [3, B, H, N, d]
    dflat = dqkv.transpose(1, 3, 0, 2, 4).reshape(B * N, 3 * H * d)
    rdw = x64.reshape(B * N, H * d).T @ dflat
    compare([("dW", to64(wd.grad), rdw)], "fp32", f"module graph copy={copy}", tol=(1e-5, 1e-5, 0))


def test_autograd_window_split_views():
    """Window-split [B, nw, H, T, d] views of a token-order qkv tensor (the
    block mask with window T) through the autograd function: the gradients
    reaching the qkv tensor, taken back to window-major order, match the
    oracle."""
    B, nw, T, H, d = 2, 5, 64, 2, 64
    q, k, v, do = make_inputs(B, H, nw * T, nw * T, d, "bf16", seed=23)
    qkv = torch.zeros((B, T, nw, 3, H, d), dtype=torch.bfloat16, device="cuda")
    for i, t in enumerate((q, k, v)):
        qkv[:, :, :, i] = t.view(B, H, nw, T, d).permute(0, 3, 2, 1, 4).cuda()
    qkv.requires_grad_(True)
    views = [qkv[:, :, :, i].permute(0, 2, 3, 1, 4) for i in range(3)]
    o = attn.fused_attention(*views)                               # [B, nw, H, T, d]
    do5 = do.cuda().view(B, H, nw, T, d).permute(0, 2, 1, 3, 4)
    (o.float() * do5.float()).sum().backward()
    torch.cuda.synchronize()
    g = qkv.grad.permute(3, 0, 4, 2, 1, 5).reshape(3, B, H, nw * T, d)   # window-major tokens
    o4 = o.permute(0, 2, 1, 3, 4).reshape(B, H, nw * T, d)
    scale = d ** -0.5
    ro, _ = oracle_fwd(to64(q), to64(k), to64(v), scale, "block", T)
    rdq, rdk, rdv = oracle_bwd(to64(q), to64(k), to64(v), to64(do), scale, "block", T)
    compare([("O", to64(o4), ro), ("dQ", to64(g[0]), rdq), ("dK", to64(g[1]), rdk),
             ("dV", to64(g[2]), rdv)], "bf16", "autograd window-split")
