"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: the whole batch runs on the GPU; the fp64 oracle then
recomputes sampled (batch, head) slices -- every head is independent, so a
slice of the inputs gives exactly that slice of every output -- and those are
compared element by element.  Over the whole output, properties that hold at
any size are checked: every value finite, rows of empty windows absent, and
the column sums of dV equal the column sums of dO per (batch, head) (rows of
P sum to one)."""
import numpy as np
import pytest
import torch

from head_attention_attn_amd.inputs import WORKLOADS, workload_inputs
from oracle import oracle_bwd, oracle_fwd

from _parity import compare, gpu_fwd_bwd, say, to64

pytestmark = pytest.mark.gpu

SAMPLES = {
    "block_local_hiera": [(0, 0), (77, 0), (127, 0)],
    "block_pooled_hiera": [(0, 0), (63, 1), (127, 1)],
    "global_vision": [(0, 0), (0, 3), (127, 2)],
    "causal_lm": [(0, 0), (0, 19)],
    "sliding_pseudo_head": [(0, 0), (0, 41), (0, 79)],
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_full_size_workload(name):
    w = WORKLOADS[name]
    say(f"[full-size] {name}: {w}")
    q, k, v, do = workload_inputs(w, seed=0)
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, w.mask, w.window, w.scale)
    say(f"[full-size] {name}: GPU done")

    # properties over the whole output
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    sdv = dv.float().sum(dim=2)
    sdo = do.cuda().float().sum(dim=2)
    rel = float((sdv - sdo).norm() / sdo.norm())
    say(f"[full-size] {name}: dV column-sum rule rel err {rel:.2e}")
    assert rel < 5e-3

    for b, h in SAMPLES[name]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        qs, ks, vs, dos = (to64(t[sl]) for t in (q, k, v, do))
        ro, rl = oracle_fwd(qs, ks, vs, w.scale, w.mask, w.window)
        rdq, rdk, rdv = oracle_bwd(qs, ks, vs, dos, w.scale, w.mask, w.window)
        rep = compare([("O", to64(o[sl]), ro), ("lse", to64(lse[sl]), rl),
                       ("dQ", to64(dq[sl]), rdq), ("dK", to64(dk[sl]), rdk),
                       ("dV", to64(dv[sl]), rdv)], w.dtype, label=f"{name} b{b} h{h}")
        say(f"[full-size] {name} b={b} h={h}: " +
            ", ".join(f"{k} {m:.2e}/{r if r is None else f'{r:.2e}'}" for k, (m, r) in rep.items()))


def test_full_size_iha_chain():
    """The interleaved-head workload at full size (20 heads, N = 8192 tokens,
    P = 4 pseudo-heads, a causal window of W = 1024 pseudo-tokens over each
    head's 32768 pseudo-tokens, d = 128; "IHA-CUDA", Pseudo-Token Mixing and
    FLOP Matching, N = 8192 row) run as the benchmark runs it: premix of Q, K,
    V, the sliding-window attention forward and backward, the premix backward.

    The oracle recomputes the chain on slices of the pseudo-token sequence.
    Under a causal window a query row depends on the W keys before it only, so
    oracle attention over the pseudo-tokens [s0, r1), with s0 = r0 - W, gives
    exactly O, lse and dQ of rows [r0, r1), and dK, dV of every key whose
    viewing queries [j, j + W) all lie in [r0, r1).  The pseudo-tokens come
    from the oracle's premix of the slice's positions, rounded to bf16 as the
    GPU stores them.  Slices at the start, the middle and the end of the
    sequence; the middle slice for every head, so that dX of the positions
    whose pseudo-tokens all have exact attention gradients is compared too.
    dW sums over every position, beyond what the oracle recomputes here; it
    is compared on the whole chain at a small size in test_gpu_premix.py."""
    import head_attention_attn_amd as attn
    from head_attention_attn_amd import binding
    from head_attention_attn_amd.inputs import make_premix_inputs
    from oracle import premix_bwd, premix_fwd

    w = WORKLOADS["iha_joint"]
    B, H, P, d, W = w.B, w.H, w.P, w.d, w.window
    N, T = w.Nq // w.P, w.Nq
    say(f"[full-size] iha_joint: B={B} H={H} N={N} P={P} d={d} W={W}")
    xs, ws = [], []
    for i in range(3):
        x, wt, dout = make_premix_inputs(B, N, H, P, d, w.dtype, seed=100 + i)
        xs.append(x)
        ws.append(wt)
    dO = dout.view(B, H, T, d)
    xd, wd = [x.cuda() for x in xs], [t.cuda() for t in ws]
    pts = [binding.premix(x, t) for x, t in zip(xd, wd)]
    q, k, v = (t.view(B, H, T, d) for t in pts)
    o, lse = attn.fwd(q, k, v, mask="sliding", window=W, scale=w.scale)
    dq, dk, dv = attn.bwd(q, k, v, o, lse, dO.cuda(), mask="sliding", window=W, scale=w.scale)
    dx = [binding.premix_bwd(x, t, g.view(B, H, N, P, d))[0] for x, t, g in zip(xd, wd, (dq, dk, dv))]
    torch.cuda.synchronize()
    say("[full-size] iha_joint: GPU done")
    for t in (o, lse, dq, dk, dv, *dx):
        assert bool(torch.isfinite(t).all())

    x64, w64 = [to64(x) for x in xs], [to64(t) for t in ws]

    def oracle_slice(r0, r1, heads):
        """Oracle chain on pseudo-tokens [s0, r1) of the given heads."""
        s0 = max(r0 - W, 0)
        n0, n1 = s0 // P, r1 // P
        ptr = [torch.tensor(premix_fwd(x[:, n0:n1], t)).to(torch.bfloat16).double().numpy()
               .reshape(B, H, (n1 - n0) * P, d) for x, t in zip(x64, w64)]
        out = {}
        for h in heads:
            qs, ks, vs = (p[:, h:h + 1] for p in ptr)
            dos = to64(dO[:, h:h + 1, s0:r1])
            ro, rl = oracle_fwd(qs, ks, vs, w.scale, "sliding", W)
            rdq, rdk, rdv = oracle_bwd(qs, ks, vs, dos, w.scale, "sliding", W)
            out[h] = (ro, rl, rdq, rdk, rdv)
        return s0, out

    mid = T // 2
    slices = [(0, 2048, [0, 11, 19]), (mid, mid + 2048, list(range(H))), (T - 2048, T, [0, 11, 19])]
    for r0, r1, heads in slices:
        s0, ref = oracle_slice(r0, r1, heads)
        kend = min(r1 - W + 1, T) if r1 < T else T  # keys whose viewers all lie in [r0, r1)
        a, kb = r0 - s0, kend - s0
        for h in heads:
            ro, rl, rdq, rdk, rdv = ref[h]
            sl = (slice(0, B), slice(h, h + 1))
            rep = compare([("O", to64(o[sl][:, :, r0:r1]), ro[:, :, a:]),
                           ("lse", to64(lse[sl][:, :, r0:r1]), rl[:, :, a:]),
                           ("dQ", to64(dq[sl][:, :, r0:r1]), rdq[:, :, a:]),
                           ("dK", to64(dk[sl][:, :, r0:kend]), rdk[:, :, a:kb]),
                           ("dV", to64(dv[sl][:, :, r0:kend]), rdv[:, :, a:kb])], w.dtype,
                          label=f"iha_joint rows [{r0},{r1}) h{h}")
            say(f"[full-size] iha_joint rows [{r0},{r1}) h={h}: " +
                ", ".join(f"{k} {m:.2e}/{r if r is None else f'{r:.2e}'}" for k, (m, r) in rep.items()))
        if len(heads) == H:
            # dX at the positions whose P pseudo-tokens all have exact
            # attention gradients in every head: pseudo-tokens [r0, kend)
            p0, p1 = -(-r0 // P), kend // P
            for i, name in enumerate("QKV"):
                g = np.concatenate([ref[h][2 + i][:, :, (p0 * P - s0):(p1 * P - s0)] for h in range(H)],
                                   axis=1).reshape(B, H, p1 - p0, P, d)
                rdx, _ = premix_bwd(x64[i][:, p0:p1], w64[i], g)
                rep = compare([(f"dX{name}", to64(dx[i][:, p0:p1]), rdx)], w.dtype,
                              label=f"iha_joint dX{name} positions [{p0},{p1})", amax_rel=2.0 ** -8)
                say(f"[full-size] iha_joint dX{name} positions [{p0},{p1}): {rep}")
