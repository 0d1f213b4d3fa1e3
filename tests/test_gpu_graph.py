"""The hot path under HIP graph capture: attn_fwd + attn_bwd (and the IHA
premix pair) captured once into a torch.cuda.CUDAGraph and replayed several
times, with new inputs copied in by eager work between the replays; every
replay must equal the eager calls on the same inputs bit for bit.  The
library allocates nothing and records no memset, so its launches are plain
kernel nodes."""
import pytest
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd import binding
from head_attention_attn_amd.inputs import make_inputs, make_premix_inputs

from _parity import say

pytestmark = pytest.mark.gpu


def _step(q, k, v, do, mask, window, keep_ds):
    o, lse = attn.fwd(q, k, v, mask=mask, window=window)
    dq, dk, dv = attn.bwd(q, k, v, o, lse, do, mask=mask, window=window, keep_ds=keep_ds)
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("B,H,N,d,mask,window,keep_ds", [
    (1, 3, 1000, 128, "causal", 0, True),      # general kernels, dS kept for the dQ pass
    (2, 2, 700, 64, "sliding", 100, False),    # general kernels, dQ recomputed
    (8, 1, 3136, 96, "block", 64, True),       # fused single-tile backward
    (16, 4, 196, 96, "none", 0, True),         # fused short-sequence backward
])
def test_graph_replays_match_eager(B, H, N, d, mask, window, keep_ds):
    say(f"[graph] {mask} B={B} H={H} N={N} d={d}")
    static = [t.cuda() for t in make_inputs(B, H, N, N, d, "bf16", seed=60)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(*static, mask, window, keep_ds)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = _step(*static, mask, window, keep_ds)
    for r in range(3):
        fresh = make_inputs(B, H, N, N, d, "bf16", seed=61 + r)
        for dst, src in zip(static, fresh):
            dst.copy_(src.cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = _step(*static, mask, window, keep_ds)
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "lse", "dQ", "dK", "dV"), outs, ref):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"
    say(f"[graph] {mask}: 3 replays equal the eager calls")


def test_graph_replays_premix():
    B, N, H, P, d = 1, 300, 20, 4, 128
    x, w, dout = (t.cuda() for t in make_premix_inputs(B, N, H, P, d, "bf16", seed=62))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.premix(x, w)
        binding.premix_bwd(x, w, dout)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = binding.premix(x, w)
        dx, dw = binding.premix_bwd(x, w, dout)
    for r in range(3):
        xf, wf, df = make_premix_inputs(B, N, H, P, d, "bf16", seed=63 + r)
        x.copy_(xf.cuda()); w.copy_(wf.cuda()); dout.copy_(df.cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ro = binding.premix(x, w)
        rdx, rdw = binding.premix_bwd(x, w, dout)
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(dx, rdx) and torch.equal(dw, rdw), f"replay {r}"
