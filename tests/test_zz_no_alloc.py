"""GPU check of attn_bwd_noalloc, the backward whose row sums live in the
library's own device scratch array (for callers that cannot allocate): called
through the C ABI, its dQ, dK, dV must equal attn_bwd's with the minimum
workspace bit for bit (the same kernels on the same inputs; bitwise equality
is stricter than the stated tolerances), on two calls in a row where the
second is smaller than the first, so that it runs over the scratch contents
the first one left."""
import pytest
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd import binding
from head_attention_attn_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

# (B, H, N, d, dtype, mask, window): a larger call, then a smaller one, per
# kernel family (general passes at d = 128 and d = 64, the fused block-local
# and short-sequence backwards, the fp32 path)
PAIRS = [
    ((2, 3, 300, 128, "bf16", "causal", 0), (1, 2, 100, 128, "bf16", "sliding", 37)),
    ((2, 2, 260, 64, "bf16", "none", 0), (1, 1, 70, 64, "bf16", "causal", 0)),
    ((4, 2, 320, 96, "bf16", "block", 64), (1, 1, 128, 96, "bf16", "block", 32)),
    ((3, 2, 196, 96, "bf16", "none", 0), (2, 1, 49, 96, "bf16", "none", 0)),
    ((1, 2, 200, 64, "fp32", "causal", 0), (1, 1, 33, 64, "fp32", "none", 0)),
]


def _run(case, seed):
    B, H, N, d, dt, mask, window = case
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in make_inputs(B, H, N, N, d, dt, seed=seed))
    kw = dict(mask=mask, window=window)
    o, lse = attn.fwd(q, k, v, **kw)
    ref = attn.bwd(q, k, v, o, lse, do, keep_ds=False, **kw)
    outs = [torch.full_like(t, float("nan")) for t in ref]
    got = binding.bwd_noalloc(q, k, v, o, lse, do, dq=outs[0], dk=outs[1], dv=outs[2], **kw)
    torch.cuda.synchronize(dev)
    print(f"noalloc case {case}", flush=True)
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert a.data_ptr() == outs[("dQ", "dK", "dV").index(name)].data_ptr()
        assert torch.equal(a, b), f"{name} differs from attn_bwd for {case}"


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_attn_bwd_twice(first, second):
    _run(first, seed=1)
    _run(second, seed=2)


def test_noalloc_refuses_rows_beyond_the_scratch():
    # 4 B H Nq bytes over 16 MiB: refused before any launch
    dev = torch.device("cuda:0")
    B, H, N, d = 1, 1, 4 * 1024 * 1024 + 256, 64
    lib = binding.load_library()
    st = lib.attn_bwd_noalloc(0, B, H, N, N, d, 0.125, 1, 0, *([None] * 9), None)
    assert st == 4  # ATTN_ERR_WORKSPACE
    torch.cuda.synchronize(dev)
