"""GPU parity of the fused backward for short key sequences (attn_bwd_fused
returns 2: at most 224 keys and 1024 query rows, d = 64 or 96, 16-bit): one
workgroup per (b, h) holds every key, so the row sums D_i, dK/dV and dQ come
out of one pass over HBM.  Against the fp64 oracle on the same seeded inputs,
for every mask, ragged key blocks (Nk not a multiple of 32) and query slabs
(Nq not a multiple of 32), Nq != Nk, and global-attention token counts of
Hiera-Base at 224x224 ("hiera-optim 0.1.0", Results: the 14x14 grid's 196
tokens, and 49 for a 7x7 grid).  The same
geometry through the three general passes, called one at a time, is checked
too: it stays reachable for callers that time or schedule the passes."""
import pytest
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd.inputs import make_inputs
from oracle import oracle_bwd, oracle_fwd

from _parity import compare, parity_case, say, to64

pytestmark = pytest.mark.gpu


def assert_short(nq, nk, d, dtype, mask, window):
    q, k, v, _ = make_inputs(1, 1, nq, nk, d, dtype, seed=0)
    kind = attn.binding.bwd_fused(q.cuda(), k.cuda(), v.cuda(), mask=mask, window=window)
    assert kind == attn.binding.FUSED_SHORT


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 96])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 37),
                                         ("sliding", 1)])
@pytest.mark.parametrize("nq,nk", [(196, 196), (49, 49), (224, 224), (1, 1), (33, 31),
                                   (300, 150), (5, 224), (100, 65)])
def test_short_matches_oracle(dtype, d, mask, window, nq, nk):
    assert_short(nq, nk, d, dtype, mask, window)
    parity_case(2, 3, nq, nk, d, dtype, mask, window, seed=50)


@pytest.mark.parametrize("d", [64, 96])
@pytest.mark.parametrize("nw,w,wq", [(4, 48, 48), (4, 48, 12), (37, 6, 3), (3, 70, 35), (1, 224, 224)])
def test_short_block_masks(d, nw, w, wq):
    """Block masks the single-tile kernels do not take (windows not dividing
    64, or longer than 64 keys), pooled or not."""
    nq, nk = nw * wq, nw * w
    assert_short(nq, nk, d, "bf16", "block", w)
    parity_case(2, 2, nq, nk, d, "bf16", "block", w, seed=51)


def test_short_many_slices():
    """More (b, h) slices than workgroups fit on the GPU at once (the global
    attention of Hiera-Base at 224^2: B = 128, 4 heads, 196 tokens), the
    first and last slices against the oracle."""
    B, H, N, d = 128, 4, 196, 96
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    q, k, v, do = make_inputs(B, H, N, N, d, "bf16", seed=52)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, lse = attn.fwd(qg, kg, vg, scale=scale)
    dq, dk, dv = attn.bwd(qg, kg, vg, o, lse, dog, scale=scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1), (77, 2)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ro, rl = oracle_fwd(to64(q[sl]), to64(k[sl]), to64(v[sl]), scale, "none", 0)
        rdq, rdk, rdv = oracle_bwd(to64(q[sl]), to64(k[sl]), to64(v[sl]), to64(do[sl]), scale,
                                   "none", 0)
        rep = compare([("dQ", to64(dq[sl]), rdq), ("dK", to64(dk[sl]), rdk),
                       ("dV", to64(dv[sl]), rdv)], "bf16", label=f"short b{b} h{h}")
        say(f"[short] b={b} h={h}: {rep}")


def test_short_deterministic():
    q, k, v, do = (t.cuda() for t in make_inputs(8, 4, 196, 196, 96, "bf16", seed=53))
    o, lse = attn.fwd(q, k, v)
    g1 = attn.bwd(q, k, v, o, lse, do)
    g2 = attn.bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


def test_short_outputs_guard_bands():
    """dQ, dK, dV written exactly: canaries around each stay."""
    B, H, nq, nk, d = 2, 2, 70, 45, 64
    q, k, v, do = (t.cuda() for t in make_inputs(B, H, nq, nk, d, "bf16", seed=54))
    o, lse = attn.fwd(q, k, v, mask="causal")
    outs = []
    for like in (q, k, v):
        n = like.numel()
        buf = torch.full((n + 2048,), 3.0, dtype=like.dtype, device="cuda")
        outs.append((buf, buf[1024:1024 + n].view(like.shape)))
    attn.bwd(q, k, v, o, lse, do, mask="causal", dq=outs[0][1], dk=outs[1][1], dv=outs[2][1])
    torch.cuda.synchronize()
    for buf, view in outs:
        n = view.numel()
        assert bool((buf[:1024] == 3.0).all()) and bool((buf[1024 + n:] == 3.0).all())


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 37)])
def test_short_geometry_through_the_general_passes(mask, window):
    """The row sums, dK/dV and dQ passes called one at a time on a short
    geometry run the general kernels; they match the oracle as well."""
    B, H, N, d = 2, 2, 200, 96
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    q, k, v, do = make_inputs(B, H, N, N, d, "bf16", seed=55)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    o, lse = attn.fwd(qg, kg, vg, mask=mask, window=window, scale=scale)
    ws = torch.empty(attn.binding.workspace_bytes(B, H, N), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    for bit in (attn.binding.PASS_ROWSUM, attn.binding.PASS_DKDV, attn.binding.PASS_DQ):
        attn.bwd(qg, kg, vg, o, lse, dog, mask=mask, window=window, scale=scale, workspace=ws,
                 dq=dq, dk=dk, dv=dv, passes=bit)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle_bwd(to64(q), to64(k), to64(v), to64(do), scale, mask, window)
    rep = compare([("dQ", to64(dq), rdq), ("dK", to64(dk), rdk), ("dV", to64(dv), rdv)], "bf16",
                  label=f"short geometry, general passes {mask}")
    say(f"[short/general] {mask}: {rep}")
