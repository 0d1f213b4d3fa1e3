"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element over whole tensors, at sizes the oracle
finishes in seconds that still span several tiles and a ragged tail.  Also the
degenerate cases, determinism, unwritten-element / out-of-bounds canaries and
large-logit stress."""
import numpy as np
import pytest
import torch

import head_attention_attn_amd as attn
from head_attention_attn_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from oracle import oracle_bwd, oracle_fwd

from _parity import compare, gpu_fwd_bwd, parity_case, say, to64

pytestmark = pytest.mark.gpu

MASKS = [("none", 0), ("causal", 0), ("sliding", 37), ("block", 16)]


def test_tiny_exact_fp32_workload():
    """The fp32 exact-check workload at its exact size: 1e-5 on every output."""
    w = WORKLOADS["tiny_exact_fp32"]
    rep = parity_case(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.mask, w.window, seed=0, scale=w.scale)
    say(f"[tiny_exact_fp32] {rep}")


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("mask,window", MASKS)
def test_bf16_ragged_multi_tile(d, mask, window):
    n = 208 if mask == "block" else 200        # 200: several 64-key tiles + a tail of 8
    parity_case(2, 2, n, n, d, "bf16", mask, window, seed=1)


@pytest.mark.parametrize("keep_ds", [True, False])
@pytest.mark.parametrize("nq,nk,mask,window", [
    (200, 200, "none", 0), (333, 333, "causal", 0), (300, 300, "sliding", 70),
    (256, 256, "block", 128),          # block mask on the general path (w does not divide 64)
    (150, 40, "sliding", 16), (37, 150, "causal", 0), (100, 37, "none", 0),
])
def test_bf16_d128_both_dq_paths(keep_ds, nq, nk, mask, window):
    """d = 128, the size where the dK/dV pass can keep dS for the dQ pass:
    with the larger workspace (dQ = scale * dS K from the kept blocks) and
    with the minimum one (dQ recomputes S and dP), each against the oracle,
    on shapes with partial key and query blocks, empty rows and Nq != Nk."""
    parity_case(2, 2, nq, nk, 128, "bf16", mask, window, seed=12, keep_ds=keep_ds)


@pytest.mark.parametrize("B,H,nq,nk,mask,window", [
    (1, 3, 260, 260, "causal", 0),
    # key blocks whose query range is empty (keys no row can see): they keep no block
    (2, 2, 37, 150, "causal", 0), (2, 2, 150, 40, "sliding", 16), (2, 2, 40, 150, "sliding", 16),
])
def test_kept_ds_workspace_guard_bands(B, H, nq, nk, mask, window):
    """The dS blocks land inside the workspace attn_bwd_workspace_size_ds
    asks for: guard bands on both sides stay untouched, and the result equals
    the recomputing path's within the bf16 tolerance."""
    d = 128
    say(f"[ds guard] {mask} W={window} bf16 d=128 B={B} H={H} Nq={nq} Nk={nk}")
    q, k, v, do = (t.cuda() for t in make_inputs(B, H, nq, nk, d, "bf16", seed=13))
    o, lse = attn.fwd(q, k, v, mask=mask, window=window)
    need = attn.binding.workspace_bytes_ds(q, k, mask=mask, window=window)
    assert need > attn.binding.workspace_bytes(B, H, nq)
    G = 1 << 16
    buf = torch.full((need + 2 * G,), 0xA5, dtype=torch.uint8, device="cuda")
    dq, dk, dv = attn.bwd(q, k, v, o, lse, do, mask=mask, window=window,
                          workspace=buf[G:G + need])
    dq2, dk2, dv2 = attn.bwd(q, k, v, o, lse, do, mask=mask, window=window, keep_ds=False)
    torch.cuda.synchronize()
    assert bool((buf[:G] == 0xA5).all()) and bool((buf[G + need:] == 0xA5).all())
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        compare([("x", to64(a), to64(b))], "bf16", "ds vs recompute")


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 5)])
def test_fp32_ragged(d, mask, window):
    parity_case(1, 2, 77, 77, d, "fp32", mask, window, seed=2)


@pytest.mark.parametrize("d", [64, 96])
@pytest.mark.parametrize("n", [1, 17, 63, 64, 65, 129])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 8)])
def test_bf16_lengths(n, mask, window, d):
    """Short sequences: one key tile taken as two 32-key halves (the second
    one empty, partial or full), a partial second tile, and a single row."""
    parity_case(1, 3, n, n, d, "bf16", mask, window, seed=n)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 96])
@pytest.mark.parametrize("n", [333, 513])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 100)])
def test_long_general_passes(d, n, mask, window, dtype):
    """d = 64, 96 past the short-sequence bounds: more than 256 keys take the
    forward's double-buffered tile loop, more than 224 the general dK/dV pass
    and the recomputing dQ pass.  Several 64-row tiles whose loads take the
    in-range path and a ragged last tile that takes the clamped one, against
    the oracle within the input type's tolerance."""
    parity_case(1, 2, n, n, d, dtype, mask, window, seed=n + d)


@pytest.mark.parametrize("nq,nk,mask,window", [
    (100, 37, "none", 0), (37, 100, "none", 0),
    (100, 37, "causal", 0), (37, 150, "causal", 0),
    (150, 40, "sliding", 16),        # rows >= 55 see no key: O = 0, lse = -inf, dQ = 0
    (40, 150, "sliding", 16),
])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_unequal_lengths_top_left(nq, nk, mask, window, dtype):
    parity_case(2, 1, nq, nk, 128 if dtype == "bf16" else 64, dtype, mask, window, seed=3)


@pytest.mark.parametrize("mask,window", [("sliding", 1), ("block", 1), ("sliding", 1000),
                                         ("block", 192), ("block", 64)])
def test_degenerate_windows(mask, window):
    """W = 1 / w = 1: each row sees only itself (O = V); W >= N is causal;
    w = N is no mask; w = 64 is the mask-unit window."""
    parity_case(2, 2, 192, 192, 96, "bf16", mask, window, seed=4)


def test_identical_keys_return_mean_value():
    """Every key equal: each row's softmax is uniform over its visible keys,
    O is the mean of those values, and dQ is exactly zero (the rows of dS sum
    to zero and multiply one common key).  rel-L2 of a zero reference is
    undefined, so dQ is held to the max-abs bound alone."""
    def same_keys(q, k, v, do):
        return q, k[:, :, :1].expand_as(k).contiguous(), v, do
    parity_case(1, 2, 130, 130, 64, "bf16", "causal", 0, seed=5, transform=same_keys,
                abs_only=("dQ",))


def _stress(q, k, v, do):
    q = (q.float() * 20).to(q.dtype)
    k = (k.float() + 3.0).to(k.dtype)
    return q, k, v, do


@pytest.mark.parametrize("dtype,d,N,mask,rel_tol,amax_frac", [
    ("bf16", 128, 300, "causal", 3e-2, 1e-2),
    ("fp32", 64, 150, "none", 1e-5, 2e-5),
])
def test_large_logits_and_key_offset(dtype, d, N, mask, rel_tol, amax_frac):
    """Q x 20 makes the softmax peaked (exercises max subtraction and the
    rescaling of the accumulator); a constant vector added to every key shifts
    each row's scores uniformly (O unchanged in exact arithmetic).

    These inputs are outside the N(0, 1) regime the tolerances are stated for,
    so the bounds here follow from each path's arithmetic, per tensor:
    rel-L2 <= rel_tol and max-abs <= amax_frac * max|ref|.
    bf16: P and dS enter their contractions rounded to bf16 (unit roundoff
    2^-8), and with the key offset the exact cancellation
    sum_j dS_ij (k_j + c) = sum_j dS_ij k_j no longer holds after rounding, so
    dQ carries an error near 2^-8 * scale * c * sum_j |dS_ij|.  Modelling
    exactly those roundings in fp64 gives rel-L2 1.9e-2 on dQ and max-abs
    <= 0.8% of each tensor's largest entry (dK reaches |49|).
    fp32: scores reach |238|, whose fp32 rounding alone (ulp 1.5e-5) moves P
    by ~1e-5 relative; plain fp32 softmax attention on the CPU lands at rel-L2
    5.3e-6 and max-abs 1.1e-5 * max|ref| on these inputs."""
    scale = float(torch.tensor(1.0 / np.sqrt(d), dtype=torch.float32))
    say(f"[stress] {dtype} {mask} N={N} d={d} Qx20 K+3")
    q, k, v, do = _stress(*make_inputs(1, 2, N, N, d, dtype, seed=6))
    o, lse, dq, dk, dv = gpu_fwd_bwd(q, k, v, do, mask, 0, scale)
    ro, rl = oracle_fwd(to64(q), to64(k), to64(v), scale, mask, 0)
    rdq, rdk, rdv = oracle_bwd(to64(q), to64(k), to64(v), to64(do), scale, mask, 0)
    for name, x, ref in (("O", o, ro), ("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        amax = amax_frac * float(np.abs(ref).max())
        rep = compare([(name, to64(x), ref)], dtype, f"stress {name}", tol=(amax, rel_tol, 0))
        say(f"[stress] {name} max-abs {rep[name][0]:.2e} rel-L2 {rep[name][1]:.2e}")
    # lse: scores of |238| carry fp32 rounding of ~1e-5 each; 1e-3 bounds it for both
    compare([("lse", to64(lse), rl)], dtype, "stress lse", tol=(0, 0, 1e-3))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("mask,window", [("causal", 0), ("none", 0), ("sliding", 300)])
def test_growing_scores_move_the_running_max(dtype, mask, window):
    """Scores that grow along the keys (about 4 log2 units per 64-key tile,
    plus one planted key whose scores jump by ~60) make the forward's running
    max move again and again inside long rows -- the rare path of its online
    softmax (rescaling O and l when a row's scores exceed the max by more
    than 2^8) -- and keep unnormalised P values up to 2^8 elsewhere.  O and
    lse against the oracle within the tolerances of the input type; the
    softmax weights are smooth (an exponential window of ~24 keys), so the
    same rounding arguments hold as for N(0, 1) inputs."""
    B, H, N, d = 1, 2, 1030, 64
    say(f"[running max] {dtype} {mask} W={window} N={N}")
    q, k, v, do = make_inputs(B, H, N, N, d, dtype, seed=12)
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    ramp = torch.arange(N, dtype=torch.float32) / N
    qf, kf = q.float() * 0.1, k.float() * 0.1
    qf[..., 0] = 16.0
    kf[..., 0] = 20.8 * ramp                  # scores rise ~0.06 log2 units per key
    kf[..., 700, 0] += 20.8                   # one key ~60 log2 units above its neighbours
    q, k = qf.to(q.dtype), kf.to(k.dtype)
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), mask=mask, window=window, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle_fwd(to64(q), to64(k), to64(v), scale, mask, window)
    rep = compare([("O", to64(o), ro), ("lse", to64(lse), rl)], dtype, f"running max {mask}")
    say(f"[running max] {rep}")


def test_deterministic_bitwise():
    say("[determinism] causal bf16 d=128 N=333")
    q, k, v, do = make_inputs(1, 4, 333, 333, 128, "bf16", seed=7)
    r1 = gpu_fwd_bwd(q, k, v, do, "causal", 0, 0.088)
    r2 = gpu_fwd_bwd(q, k, v, do, "causal", 0, 0.088)
    for a, b in zip(r1, r2):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                           b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_poison_and_guard_bands(dtype):
    """Outputs pre-filled with NaN must be fully overwritten; guard bands
    around every output must stay untouched."""
    B, H, N, d = 2, 2, 150, 96
    say(f"[canary] {dtype}")
    q, k, v, do = (t.cuda() for t in make_inputs(B, H, N, N, d, dtype, seed=8))
    tdt = q.dtype
    G = 4096  # guard elements on each side

    def guarded(shape, dt):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * G,), float("nan"), dtype=dt, device="cuda")
        return buf, buf[G:G + n].view(shape)

    def guards_ok(buf, n):
        return bool(torch.isnan(buf[:G]).all()) and bool(torch.isnan(buf[G + n:]).all())

    ob, o = guarded((B, H, N, d), tdt)
    lb, lse = guarded((B, H, N), torch.float32)
    attn.fwd(q, k, v, mask="sliding", window=40, out=o, lse=lse)
    bufs = [guarded((B, H, N, d), tdt) for _ in range(3)]
    wsb, ws = guarded((attn.binding.workspace_bytes(B, H, N) // 4,), torch.float32)
    attn.bwd(q, k, v, o, lse, do, mask="sliding", window=40, workspace=ws.view(torch.uint8),
             dq=bufs[0][1], dk=bufs[1][1], dv=bufs[2][1])
    torch.cuda.synchronize()
    for t in (o, lse, bufs[0][1], bufs[1][1], bufs[2][1]):
        assert not torch.isnan(t).any()
    n4 = B * H * N * d
    assert guards_ok(ob, n4) and guards_ok(lb, B * H * N) and guards_ok(wsb, ws.numel())
    for buf, _ in bufs:
        assert guards_ok(buf, n4)
    ro, rl = oracle_fwd(to64(q), to64(k), to64(v), 1 / np.sqrt(d), "sliding", 40)
    compare([("O", to64(o), ro), ("lse", to64(lse), rl)], dtype, "canary")


def test_error_paths_leave_outputs_untouched():
    q, k, v, _ = (t.cuda() for t in make_inputs(1, 1, 64, 64, 64, "bf16", seed=9))
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 1, 64), 7.0, device="cuda")
    with pytest.raises(attn.AttnError) as ei:
        attn.fwd(q, k, v, mask="block", window=5, out=o, lse=lse)      # 64 % 5 != 0
    assert ei.value.status == 1
    with pytest.raises(attn.AttnError) as ei:
        attn.fwd(q, k, v, out=q, lse=lse)                              # output aliases input
    assert ei.value.status == 5
    torch.cuda.synchronize()
    assert bool((o == 7).all()) and bool((lse == 7).all())


def test_binding_rejects_mismatched_outputs():
    """Caller-provided outputs of the wrong dtype, shape, device or layout are
    refused before any launch (the library writes B * H * Nq floats at lse's
    base and whole rows at the others')."""
    q, k, v, do = (t.cuda() for t in make_inputs(1, 2, 64, 64, 64, "bf16", seed=9))
    bad = [dict(out=torch.empty(1, 2, 64, 64, device="cuda")),                    # fp32 O
           dict(out=torch.empty(1, 2, 32, 64, dtype=torch.bfloat16, device="cuda")),
           dict(lse=torch.empty(1, 2, 32, device="cuda")),                        # short lse
           dict(lse=torch.empty(1, 2, 64, dtype=torch.float64, device="cuda")),
           dict(lse=torch.empty(1, 64, 2, device="cuda").transpose(1, 2))]        # strided lse
    for kw in bad:
        with pytest.raises(ValueError):
            attn.fwd(q, k, v, mask="causal", **kw)
    o, lse = attn.fwd(q, k, v, mask="causal")
    for kw in (dict(dq=torch.empty(1, 2, 64, 32, dtype=torch.bfloat16, device="cuda")),
               dict(dk=torch.empty(1, 2, 64, 64, device="cuda")),
               dict(dv=torch.empty(1, 2, 64, 64, dtype=torch.bfloat16))):
        with pytest.raises(ValueError):
            attn.bwd(q, k, v, o, lse, do, mask="causal", **kw)
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, lse[:, :, :32], do, mask="causal")
    torch.cuda.synchronize()


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("window,n", [(64, 192), (32, 96), (16, 208), (8, 40), (4, 12), (2, 130),
                                      (1, 65)])
def test_block_local_single_tile_path(d, window, n):
    """Block-local windows dividing 64 take the single-tile kernels (fused
    backward); n not a multiple of 64 leaves a partial last tile.

    With windows of 1-4 keys the softmax barely averages, so dV (a sum of up
    to w rows of dO) reaches |5|, where the bf16 rounding of the output alone
    is up to 2^-8 * |x| = 0.02: the max-abs bound grows by 2^-8 * max|ref|
    for those windows.  rel-L2 keeps the 5e-3 bound."""
    B, H = 3, 2
    q, k, v, _ = make_inputs(B, H, n, n, d, "bf16", seed=10)
    assert attn.binding.bwd_fused(q.cuda(), k.cuda(), v.cuda(), mask="block", window=window)
    parity_case(B, H, n, n, d, "bf16", "block", window, seed=10,
                amax_rel=2.0 ** -8 if window <= 4 else 0.0)


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("nw,w,wq,single_tile", [
    (5, 48, 12, False),   # 60 query rows over 240 keys: one partial query tile
    (7, 40, 10, False),   # windows straddle 64-key tiles
    (37, 6, 3, False),    # 111 queries, 222 keys: ragged tails on both sides
    (9, 64, 16, True),    # Hiera's q_stride 4: 16 query rows per 64-key tile
    (11, 32, 16, True),   # 32 rows per tile, partial last tile (352 keys)
    (13, 16, 1, True),    # one pooled query per window, 4 rows per tile
    (7, 8, 4, True),      # 56 keys: one partial tile of 28 rows
    (5, 64, 32, True),    # q_stride 2
    (3, 64, 64, True),    # no pooling, 64-key windows
])
def test_block_pooled_queries(d, nw, w, wq, single_tile):
    """Block mask with pooled queries: Nk / w windows of w keys each hold
    Nq / (Nk / w) = wq query rows (Hiera's q_stride = w / wq).  Key windows
    dividing 64 with wq dividing w run as single tiles (64 keys and their
    64 wq / w query rows), the rest on the fused short-sequence kernel (at
    most 224 keys, d <= 96) or the general kernels."""
    nq, nk = nw * wq, nw * w
    q, k, v, _ = make_inputs(1, 1, nq, nk, d, "bf16", seed=14)
    kind = (attn.binding.FUSED_LOCAL if single_tile else
            attn.binding.FUSED_SHORT if nk <= 224 and d <= 96 else 0)
    assert attn.binding.bwd_fused(q.cuda(), k.cuda(), v.cuda(), mask="block", window=w) == kind
    parity_case(2, 2, nq, nk, d, "bf16", "block", w, seed=14)


@pytest.mark.parametrize("keep_ds", [True, False])
def test_block_pooled_d128_both_dq_paths(keep_ds):
    """Pooled block mask at d = 128 with and without the kept-dS dQ pass."""
    parity_case(2, 2, 13 * 24, 13 * 96, 128, "bf16", "block", 96, seed=15, keep_ds=keep_ds)


def test_block_pooled_fp32():
    parity_case(2, 2, 9 * 8, 9 * 32, 64, "fp32", "block", 32, seed=16)


def test_fused_backward_rejects_partial_pass_sets():
    q, k, v, do = (t.cuda() for t in make_inputs(1, 1, 128, 128, 96, "bf16", seed=11))
    o, lse = attn.fwd(q, k, v, mask="block", window=64)
    with pytest.raises(attn.AttnError) as ei:
        attn.bwd(q, k, v, o, lse, do, mask="block", window=64, passes=attn.binding.PASS_DKDV)
    assert ei.value.status == 2
