"""GPU parity of fp16 inputs (ATTN_FP16): the 16-bit kernels with the fp16
MFMA (v_mfma_f32_32x32x16_f16), P and dS rounded to fp16, outputs rounded to
fp16 -- against the fp64 oracle on the same seeded inputs (rounded to fp16 by
the input generator), within the fp16 tolerance of tests/_parity.py.  The
pages' Hiera test matrix runs bf16, fp16 and fp32 ("hiera-optim 0.1.0",
Tests)."""
import pytest
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from oracle import oracle_bwd, oracle_fwd

from _parity import compare, gpu_fwd_bwd, parity_case, say, to64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 37), ("block", 16)])
def test_fp16_ragged_multi_tile(d, mask, window):
    n = 208 if mask == "block" else 200
    parity_case(2, 2, n, n, d, "fp16", mask, window, seed=30)


@pytest.mark.parametrize("keep_ds", [True, False])
@pytest.mark.parametrize("nq,nk,mask,window", [
    (333, 333, "causal", 0), (150, 40, "sliding", 16), (37, 150, "causal", 0),
    (13 * 24, 13 * 96, "block", 96),
])
def test_fp16_d128_both_dq_paths(keep_ds, nq, nk, mask, window):
    """d = 128: dQ from dS kept (in fp16) by the dK/dV pass, or recomputed."""
    parity_case(2, 2, nq, nk, 128, "fp16", mask, window, seed=31, keep_ds=keep_ds)


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("nw,w,wq", [(3, 64, 64), (13, 16, 16), (9, 64, 16), (11, 32, 16)])
def test_fp16_single_tile(d, nw, w, wq):
    """Block-local windows on the single-tile kernels, pooled or not."""
    q, k, v, _ = make_inputs(1, 1, nw * wq, nw * w, d, "fp16", seed=32)
    assert attn.binding.bwd_fused(q.cuda(), k.cuda(), v.cuda(), mask="block", window=w)
    parity_case(3, 2, nw * wq, nw * w, d, "fp16", "block", w, seed=32)


def test_fp16_strided_sequence_major():
    """fp16 tensors as [B, N, H, d] buffers viewed as [B, H, N, d]: bitwise
    equal to the contiguous call."""
    B, H, N, d = 2, 3, 150, 96
    q, k, v, do = (t.cuda() for t in make_inputs(B, H, N, N, d, "fp16", seed=33))
    qs, ks, vs, dos = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v, do))
    assert not qs.is_contiguous()
    o, lse = attn.fwd(qs, ks, vs, mask="causal")
    g = attn.bwd(qs, ks, vs, o, lse, dos, mask="causal")
    oc, lc = attn.fwd(q, k, v, mask="causal")
    gc = attn.bwd(q, k, v, oc, lc, do, mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    assert all(torch.equal(a, b) for a, b in zip(g, gc))


def test_fp16_full_size_block_local():
    """The Hiera mask-unit workload in fp16 at its full size (B=128, 3136
    tokens, 49 windows of 64, d=96), sampled (batch, head) slices against the
    oracle."""
    w = WORKLOADS["block_local_hiera"]
    say(f"[fp16 full-size] {w}")
    q, k, v, do = make_inputs(w.B, w.H, w.Nq, w.Nk, w.d, "fp16", seed=0)
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, w.mask, w.window, w.scale)
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    for b in (0, 64, 127):
        sl = (slice(b, b + 1), slice(0, 1))
        qs, ks, vs, dos = (to64(t[sl]) for t in (q, k, v, do))
        ro, rl = oracle_fwd(qs, ks, vs, w.scale, w.mask, w.window)
        rdq, rdk, rdv = oracle_bwd(qs, ks, vs, dos, w.scale, w.mask, w.window)
        rep = compare([("O", to64(o[sl]), ro), ("lse", to64(lse[sl]), rl),
                       ("dQ", to64(dq[sl]), rdq), ("dK", to64(dk[sl]), rdk),
                       ("dV", to64(dv[sl]), rdv)], "fp16", label=f"fp16 full b{b}")
        say(f"[fp16 full-size] b={b}: {rep}")
