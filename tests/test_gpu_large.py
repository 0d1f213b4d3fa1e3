"""GPU parity past 2^31 elements per tensor: slice offsets beyond 32 bits on
the general kernels (sliding window, d = 128, kept dS) and on the fused
single-tile kernels (Hiera mask units, d = 96).  Inputs are drawn on the
device (inputs.make_device_inputs); the oracle checks the slices at the far
end of each tensor, whose elements sit past 2^31, on the rows and keys whose
whole visible windows lie inside the checked slice."""
import pytest
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd.inputs import make_device_inputs
from oracle import oracle_bwd, oracle_fwd

from _parity import compare, gpu_fwd_bwd, say, to64

pytestmark = pytest.mark.gpu


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_sliding_window_past_2_31_elements():
    B, H, N, d, W = 1, 3, 5_600_000, 128, 64
    assert B * H * N * d > 2 ** 31 and N * d <= 2 ** 31
    say(f"[large] sliding B={B} H={H} N={N} d={d} W={W}: {B * H * N * d / 2 ** 31:.2f} x 2^31 elements")
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    q, k, v, do = make_device_inputs(B, H, N, N, d, "bf16", seed=50)
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, "sliding", W, scale, keep_ds=True)
    # the last 320 rows of the last head: rows / keys >= N - 256 have their
    # whole window inside it
    s0, c0 = N - 320, 64
    sl = (slice(B - 1, B), slice(H - 1, H), slice(s0, N))
    qs, ks, vs, dos = (to64(t[sl]) for t in (q, k, v, do))
    ro, rl = oracle_fwd(qs, ks, vs, scale, "sliding", W)
    rdq, rdk, rdv = oracle_bwd(qs, ks, vs, dos, scale, "sliding", W)
    tail = (slice(None), slice(None), slice(c0, None))
    rep = compare([("O", to64(o[sl])[tail], ro[tail]), ("lse", to64(lse[sl[:3]])[tail], rl[tail]),
                   ("dQ", to64(dq[sl])[tail], rdq[tail]), ("dK", to64(dk[sl])[tail], rdk[tail]),
                   ("dV", to64(dv[sl])[tail], rdv[tail])], "bf16", label="large sliding")
    say(f"[large] sliding {rep}")
    del q, k, v, do, o, lse, dq, dk, dv
    _free()


def test_block_local_past_2_31_elements():
    B, H, N, d, w = 7200, 1, 3136, 96, 64
    assert B * H * N * d > 2 ** 31
    say(f"[large] block-local B={B} N={N} d={d}: {B * H * N * d / 2 ** 31:.2f} x 2^31 elements")
    q, k, v, do = make_device_inputs(B, H, N, N, d, "bf16", seed=51)
    assert attn.binding.bwd_fused(q, k, v, mask="block", window=w)
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, "block", w, scale)
    for b in (B - 1, (2 ** 31) // (N * d) + 1):       # both slices start past 2^31 elements
        assert b * N * d > 2 ** 31
        sl = (slice(b, b + 1), slice(0, 1))
        qs, ks, vs, dos = (to64(t[sl]) for t in (q, k, v, do))
        ro, rl = oracle_fwd(qs, ks, vs, scale, "block", w)
        rdq, rdk, rdv = oracle_bwd(qs, ks, vs, dos, scale, "block", w)
        rep = compare([("O", to64(o[sl]), ro), ("lse", to64(lse[sl]), rl), ("dQ", to64(dq[sl]), rdq),
                       ("dK", to64(dk[sl]), rdk), ("dV", to64(dv[sl]), rdv)], "bf16",
                      label=f"large block b{b}")
        say(f"[large] block b={b}: {rep}")
    del q, k, v, do, o, lse, dq, dk, dv
    _free()
