"""GPU parity of the IHA premix kernels (attn_premix_fwd / attn_premix_bwd)
against the fp64 oracle (oracle/premix.py) on the same seeded inputs, and of
the whole interleaved-head-attention chain (premix of Q, K, V -> sliding
window attention over the pseudo-tokens -> backward through both).

Bounds, element by element, from the arithmetic: the fp32 sum s of n
products is within n 2^-24 sum |terms| of the exact value ref, and rounding
s to nearest even in 16 bits adds at most u |s| <= u (|ref| + |s - ref|), so
the output is within u |ref| + (1 + u) n 2^-24 sum |terms| of ref (u = 2^-8
for bf16, 2^-11 for fp16); dW is fp32
(a blocked sum over B * N * d products): within depth * 2^-24 sum |terms|, with
depth the longest chain of additions of the blocking (``dw_depth``).  In the chained test the gradients reaching
the inputs are products of the attention gradients (bf16 tolerance) and W,
so their max-abs bound grows by the output rounding 2^-8 max |ref| as for
other large-magnitude results."""
import numpy as np
import pytest
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd import binding
from head_attention_attn_amd.inputs import make_premix_inputs
from oracle import oracle_bwd, oracle_fwd
from oracle.premix import premix_bwd, premix_fwd

from _parity import compare, say, to64

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def check_elementwise(name, got, ref, absref, u, nterms):
    bound = u * np.abs(ref) + (1 + u) * (nterms * 2.0 ** -24 + 1e-30) * absref + 1e-7
    err = np.abs(got - ref)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"{name}: error {worst:.2f} x its bound"
    return worst


def dw_depth(npos, d):
    """Longest chain of fp32 additions behind one dW element: a workgroup's
    positions times a wave's 32 features, the d / 32 waves, then the 16-way
    and 16-deep reduction over the min(npos, 1024) workgroup partials."""
    grid = min(npos, 1024)
    return -(-npos // grid) * 32 + d // 32 + -(-grid // 16) + 16


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("B,N,H,P,d", [
    (2, 37, 20, 4, 128),     # the IHA LLaMA head count and pseudo-heads, ragged N
    (1, 50, 3, 2, 64),
    (2, 9, 32, 4, 96),       # 32 source heads, 128 pseudo-heads: every tile full
    (1, 1, 1, 1, 64),
    (3, 17, 7, 8, 128),      # 56 pseudo-heads: partial tiles and k-steps
    (1, 1100, 5, 4, 64),     # more positions than workgroups (1024)
])
def test_premix_matches_oracle(dtype, B, N, H, P, d):
    say(f"[premix] {dtype} B={B} N={N} H={H} P={P} d={d}")
    x, w, dout = make_premix_inputs(B, N, H, P, d, dtype, seed=40)
    xg, wg, dg = x.cuda(), w.cuda(), dout.cuda()
    out = binding.premix(xg, wg)
    dx, dw = binding.premix_bwd(xg, wg, dg)
    torch.cuda.synchronize()
    x64, w64, d64 = to64(x), to64(w), to64(dout)
    ref = premix_fwd(x64, w64)
    absref = premix_fwd(np.abs(x64), np.abs(w64))
    rdx, rdw = premix_bwd(x64, w64, d64)
    adx, adw = premix_bwd(np.abs(x64), np.abs(w64), np.abs(d64))
    r = [check_elementwise("out", to64(out), ref, absref, U[dtype], H),
         check_elementwise("dx", to64(dx), rdx, adx, U[dtype], H * P),
         check_elementwise("dw", to64(dw), rdw, adw, 0.0, dw_depth(B * N, d))]
    say(f"[premix] worst error / bound: out {r[0]:.3f} dx {r[1]:.3f} dw {r[2]:.3f}")


def test_premix_deterministic():
    x, w, dout = (t.cuda() for t in make_premix_inputs(1, 3000, 20, 4, 128, "bf16", seed=41))
    a = binding.premix(x, w)
    g1 = binding.premix_bwd(x, w, dout)
    b = binding.premix(x, w)
    g2 = binding.premix_bwd(x, w, dout)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1])


def test_premix_output_guard_bands():
    """The output is written exactly: canaries around it stay."""
    B, N, H, P, d = 1, 40, 6, 4, 64
    x, w, _ = (t.cuda() for t in make_premix_inputs(B, N, H, P, d, "bf16", seed=42))
    n = B * H * N * P * d
    buf = torch.full((n + 2048,), 3.0, dtype=torch.bfloat16, device="cuda")
    out = buf[1024:1024 + n].view(B, H, N, P, d)
    binding.premix(x, w, out=out)
    torch.cuda.synchronize()
    assert bool((buf[:1024] == 3.0).all()) and bool((buf[1024 + n:] == 3.0).all())


def test_iha_chain_matches_oracle():
    """Interleaved head attention end to end: pseudo-tokens of Q, K, V by the
    premix, causal sliding-window attention of W pseudo-tokens over each
    head's N * P pseudo-tokens (the joint softmax across pseudo-heads), and
    gradients back to the inputs and the mixing weights through the autograd
    wrappers -- against the oracle's premix and attention chained the same
    way."""
    B, N, H, P, d, W = 1, 48, 4, 4, 64, 40
    scale = d ** -0.5
    xs, ws, dos = [], [], None
    for i in range(3):
        x, w, dout = make_premix_inputs(B, N, H, P, d, "bf16", seed=43 + i)
        xs.append(x)
        ws.append(w)
        dos = dout.view(B, H, N * P, d)
    xg = [x.cuda().requires_grad_(True) for x in xs]
    wg = [w.cuda().requires_grad_(True) for w in ws]
    o = attn.iha_attention(*xg, *wg, window=W, scale=scale)
    (o.float() * dos.cuda().float()).sum().backward()
    torch.cuda.synchronize()
    # oracle: premix -> attention -> gradients chained by hand
    x64 = [to64(x) for x in xs]
    w64 = [to64(w) for w in ws]
    # pseudo-tokens rounded to bf16 as the GPU path stores them
    pt = [torch.tensor(premix_fwd(x, w)).to(torch.bfloat16).double().numpy()
          .reshape(B, H, N * P, d) for x, w in zip(x64, w64)]
    ro, _ = oracle_fwd(*pt, scale, "sliding", W)
    rdq, rdk, rdv = oracle_bwd(*pt, to64(dos), scale, "sliding", W)
    refs = []
    for x, w, g in zip(x64, w64, (rdq, rdk, rdv)):
        refs.append(premix_bwd(x, w, g.reshape(B, H, N, P, d)))
    compare([("O", to64(o), ro)], "bf16", "iha chain O")
    for i, name in enumerate("qkv"):
        rdx, rdw = refs[i]
        compare([(f"dX{name}", to64(xg[i].grad), rdx)], "bf16", f"iha chain dX{name}",
                amax_rel=2.0 ** -8)
        compare([(f"dW{name}", to64(wg[i].grad), rdw)], "bf16", f"iha chain dW{name}",
                amax_rel=2.0 ** -8)
