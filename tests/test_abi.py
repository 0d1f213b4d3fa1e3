"""The C-ABI library on the CPU: it loads, exports every entry point that
include/attn.h declares, and its argument validation returns the documented
status codes (attn_check_* make no device call, so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

from head_attention_attn_amd import binding
from oracle.attention import visible

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, ALIAS, DEVICE, LAUNCH = range(8)
BF16, FP32, FP16 = 0, 1, 2
MASK = {"none": 0, "causal": 1, "sliding": 2, "block": 3}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.lib_path()):
        from head_attention_attn_amd.build import build
        build()
    return binding.load_library()


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    return sorted(set(re.findall(r"ATTN_API\s+[\w\s\*]+?\b(attn_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == sorted(["attn_fwd", "attn_bwd", "attn_bwd_passes", "attn_bwd_fused",
                                         "attn_bwd_workspace_size", "attn_bwd_workspace_size_ds",
                                         "attn_check_fwd", "attn_check_bwd", "attn_status_string",
                                         "attn_layouts_contiguous", "attn_fwd_strided",
                                         "attn_bwd_strided", "attn_check_fwd_strided",
                                         "attn_check_bwd_strided", "attn_premix_fwd",
                                         "attn_premix_bwd", "attn_premix_bwd_workspace_size",
                                         "attn_check_premix_fwd", "attn_check_premix_bwd",
                                         "attn_bwd_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.lib_path()],
                         capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(declared_symbols()) <= exported
    # nothing else of ours leaks out of the shared object
    assert not [s for s in exported if s.startswith("_ZN4attn")]


def test_status_strings(lib):
    names = ["ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_MISALIGNED",
             "ATTN_ERR_WORKSPACE", "ATTN_ERR_ALIAS", "ATTN_ERR_DEVICE", "ATTN_ERR_LAUNCH"]
    for code, name in enumerate(names):
        assert lib.attn_status_string(code).decode() == name
    assert lib.attn_status_string(99).decode() == "ATTN_ERR_UNKNOWN"


def test_workspace_size(lib):
    assert lib.attn_bwd_workspace_size(1, 1, 1) == 256
    assert lib.attn_bwd_workspace_size(1, 20, 8192) == 20 * 8192 * 4
    assert lib.attn_bwd_workspace_size(3, 1, 5) == 256
    assert lib.attn_bwd_workspace_size(0, 1, 5) == 0


def _ds_blocks_from_visibility(mask, window, nq, nk):
    """32 x 32 (key block, query block) pairs holding a visible entry, counted
    from the oracle's visibility matrix."""
    vis = visible(mask, window, nq, nk)
    n = 0
    for kb in range(0, nk, 32):
        for jb in range(0, nq, 32):
            n += bool(vis[jb:jb + 32, kb:kb + 32].any())
    return n


@pytest.mark.parametrize("nq,nk,mask,window", [
    (128, 128, "causal", 0), (333, 333, "causal", 0), (200, 200, "none", 0),
    (300, 300, "sliding", 70), (256, 256, "block", 128), (150, 40, "sliding", 16),
    (37, 150, "causal", 0), (100, 37, "none", 0), (40, 150, "sliding", 16),
    (96, 384, "block", 96), (100, 200, "block", 40),      # pooled queries
])
def test_workspace_size_ds_counts_visible_blocks(lib, nq, nk, mask, window):
    """attn_bwd_workspace_size_ds = row sums + 2 KB per visible 32 x 32
    block per (b, h), the blocks counted here independently of the library."""
    B, H = 2, 3
    base = lib.attn_bwd_workspace_size(B, H, nq)
    got = lib.attn_bwd_workspace_size_ds(0, B, H, nq, nk, 128, MASK[mask], window)
    assert got == base + B * H * _ds_blocks_from_visibility(mask, window, nq, nk) * 2048


def test_pooled_block_single_tile_dispatch(lib):
    """Key windows dividing 64 whose query windows divide them run as single
    tiles (fused backward, 1), pooled or not; other block shapes with at
    most 224 keys take the short-sequence fused backward (2), longer ones
    the general passes (0)."""
    assert lib.attn_bwd_fused(0, 1, 1, 3136, 3136, 96, 3, 64) == 1
    assert lib.attn_bwd_fused(0, 1, 1, 784, 3136, 96, 3, 64) == 1     # 16 query rows per window
    assert lib.attn_bwd_fused(0, 1, 1, 4, 64, 96, 3, 16) == 1         # one query row per window
    assert lib.attn_bwd_fused(0, 1, 1, 12, 64, 96, 3, 16) == 2        # 3 rows per window of 16
    assert lib.attn_bwd_fused(0, 1, 1, 20, 80, 96, 3, 80) == 2        # window 80 does not divide 64
    assert lib.attn_bwd_fused(0, 1, 1, 60, 240, 96, 3, 80) == 0       # ... 240 keys
    assert lib.attn_bwd_fused(1, 1, 1, 784, 3136, 96, 3, 64) == 0     # fp32
    assert lib.attn_bwd_fused(2, 1, 1, 784, 3136, 96, 3, 64) == 1     # fp16
    assert lib.attn_bwd_fused(0, 1, 1, 15, 64, 96, 3, 16) == 0        # invalid: 4 windows, 15 rows


def test_workspace_size_ds_where_it_does_not_apply(lib):
    base = lib.attn_bwd_workspace_size(1, 2, 256)
    assert lib.attn_bwd_workspace_size_ds(0, 1, 2, 256, 256, 96, 1, 0) == base     # d != 128
    assert lib.attn_bwd_workspace_size_ds(1, 1, 2, 256, 256, 128, 1, 0) == base    # fp32
    assert lib.attn_bwd_workspace_size_ds(2, 1, 2, 256, 256, 128, 1, 0) > base     # fp16 keeps dS
    assert lib.attn_bwd_workspace_size_ds(0, 1, 2, 256, 256, 128, 3, 64) == base   # fused block-local
    assert lib.attn_bwd_workspace_size_ds(0, 1, 2, 256, 256, 128, 3, 5) == 0       # invalid window
    # the causal N=8192, H=20 workload: 256 * 257 / 2 blocks per head
    assert lib.attn_bwd_workspace_size_ds(0, 1, 20, 8192, 8192, 128, 1, 0) == \
        lib.attn_bwd_workspace_size(1, 20, 8192) + 20 * (256 * 257 // 2) * 2048


# Fake, never-dereferenced device addresses, far apart and 16-byte aligned.
BASE = 1 << 40
STEP = 1 << 32


def ptrs(n):
    return [BASE + i * STEP for i in range(n)]


def fwd_args(**kw):
    a = dict(dtype=BF16, B=2, H=3, Nq=100, Nk=100, d=64, scale=0.125, mask=0, window=0)
    q, k, v, o, lse = ptrs(5)
    a.update(q=q, k=k, v=v, o=o, lse=lse)
    a.update(kw)
    return a


def check_fwd(lib, **kw):
    a = fwd_args(**kw)
    return lib.attn_check_fwd(a["dtype"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"],
                              a["mask"], a["window"], a["q"], a["k"], a["v"], a["o"], a["lse"])


def check_bwd(lib, ws_bytes=None, **kw):
    a = fwd_args(**kw)
    p = ptrs(11)
    names = ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "ws"]
    b = {n: p[i] for i, n in enumerate(names)}
    b.update({k: v for k, v in kw.items() if k in names})
    ws = lib.attn_bwd_workspace_size(a["B"], a["H"], a["Nq"]) if ws_bytes is None else ws_bytes
    return lib.attn_check_bwd(a["dtype"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"],
                              a["mask"], a["window"], b["q"], b["k"], b["v"], b["o"], b["lse"],
                              b["dout"], b["dq"], b["dk"], b["dv"], b["ws"], ws)


def test_valid_arguments_pass(lib):
    for mask, window in ((0, 0), (1, 0), (2, 1024), (3, 4)):
        assert check_fwd(lib, mask=mask, window=window) == OK
        assert check_bwd(lib, mask=mask, window=window) == OK
    assert check_fwd(lib, dtype=FP32, d=96) == OK
    assert check_fwd(lib, dtype=FP16, d=128) == OK
    assert check_bwd(lib, dtype=FP16, mask=1) == OK
    assert check_fwd(lib, Nq=7, Nk=300, mask=1) == OK          # Nq != Nk, top-left causal
    assert check_fwd(lib, Nq=50, Nk=100, mask=3, window=4) == OK  # pooled: 25 windows of 2 rows x 4 keys


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), UNSUPPORTED),
    (dict(dtype=-1), UNSUPPORTED),
    (dict(d=80), UNSUPPORTED),
    (dict(d=256), UNSUPPORTED),
    (dict(B=0), INVALID),
    (dict(H=-1), INVALID),
    (dict(Nq=0), INVALID),
    (dict(Nk=0), INVALID),
    (dict(mask=4), INVALID),
    (dict(mask=-1), INVALID),
    (dict(mask=2, window=0), INVALID),
    (dict(mask=3, window=0), INVALID),
    (dict(mask=3, window=7), INVALID),            # 100 % 7 != 0
    (dict(mask=3, window=4, Nk=96), INVALID),     # 24 windows do not divide Nq = 100
    (dict(mask=3, window=4, Nq=24, Nk=100), INVALID),  # 25 windows do not divide Nq = 24
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(q=0), INVALID),
    (dict(lse=0), INVALID),
    (dict(k=BASE + 8), MISALIGNED),
    (dict(o=BASE + 20 * STEP + 4), MISALIGNED),
    (dict(o=BASE), ALIAS),                                   # output == input
    (dict(lse=BASE + 3 * STEP + 1024), ALIAS),               # lse inside o
    (dict(Nq=1 << 31), INVALID),
])
def test_fwd_validation(lib, kw, status):
    assert check_fwd(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(ws=0), WORKSPACE),
    (dict(ws_bytes=16), WORKSPACE),
    (dict(dq=BASE), ALIAS),
    (dict(dv=BASE + 6 * STEP + 64), ALIAS),        # dv inside dq
    (dict(ws=BASE + 5 * STEP), ALIAS),             # workspace on top of dout
    (dict(dout=BASE + 5 * STEP + 2), MISALIGNED),
    (dict(dk=0), INVALID),
    (dict(d=48), UNSUPPORTED),
])
def test_bwd_validation(lib, kw, status):
    assert check_bwd(lib, **kw) == status


def test_fused_backward_predicate(lib):
    """The backward is one fused kernel for 16-bit block-local attention whose
    window divides 64 (1) and for 16-bit attention with at most 224 keys and
    1024 query rows at d = 64 or 96 (2); invalid geometry reports 0."""
    f = lambda dtype, n, mask, w, d=96, nq=None: lib.attn_bwd_fused(
        dtype, 2, 1, n if nq is None else nq, n, d, mask, w)
    for w in (1, 2, 4, 8, 16, 32, 64):
        assert f(BF16, 3136, 3, w) == 1
        assert f(FP16, 3136, 3, w) == 1
    assert f(BF16, 3136, 3, 7 * 64) == 0        # window 448 > 64
    assert f(BF16, 192, 3, 48) == 2             # 48 does not divide 64; 192 keys
    assert f(BF16, 960, 3, 48) == 0             # ... 960 keys
    for mask, w in ((0, 0), (1, 0), (2, 37)):
        assert f(BF16, 196, mask, w) == 2       # short sequences, any mask
        assert f(FP16, 224, mask, w, d=64) == 2
        assert f(BF16, 225, mask, w) == 0       # 225 keys
        assert f(BF16, 196, mask, w, d=128) == 0
        assert f(FP32, 196, mask, w) == 0
    assert f(BF16, 100, 0, 0, nq=1024) == 2
    assert f(BF16, 100, 0, 0, nq=1025) == 0     # long query sequence
    assert f(FP32, 3136, 3, 64) == 0            # fp32 path is not fused
    assert f(BF16, 3136, 0, 64) == 0            # mask none
    assert f(BF16, 3136, 2, 64) == 0            # sliding
    assert f(BF16, 100, 3, 64) == 0             # 100 % 64 != 0: invalid geometry
    assert f(BF16, 128, 3, 64, d=80) == 0       # unsupported d


def test_premix_validation(lib):
    B, N, H, P, d = 1, 64, 20, 4, 128
    x, w, out, dout, dx, dw, ws = ptrs(7)
    ck = lambda dtype=BF16, **kw: lib.attn_check_premix_fwd(
        dtype, kw.get("B", B), kw.get("N", N), kw.get("H", H), kw.get("P", P), kw.get("d", d),
        kw.get("x", x), kw.get("w", w), kw.get("out", out))
    assert ck() == OK
    assert ck(FP16) == OK
    assert ck(FP32) == UNSUPPORTED                       # 16-bit MFMA path only
    assert ck(H=33) == UNSUPPORTED and ck(H=20, P=8) == UNSUPPORTED and ck(P=3) == UNSUPPORTED
    assert ck(d=80) == UNSUPPORTED
    assert ck(N=0) == INVALID and ck(x=0) == INVALID
    assert ck(N=1 << 20, H=32, P=4) == INVALID           # H*N*P*d >= 2^31
    assert ck(w=BASE + 8) == MISALIGNED
    assert ck(out=x + 128) == ALIAS                      # output inside x
    wsz = lib.attn_premix_bwd_workspace_size(B, N, H, P)
    assert wsz == ((min(B * N, 1024) * H * P * H * 4 + 255) // 256) * 256
    assert lib.attn_premix_bwd_workspace_size(4, 8192, H, P) == 1024 * H * P * H * 4
    assert lib.attn_premix_bwd_workspace_size(1, 1, 33, 1) == 0
    cb = lambda **kw: lib.attn_check_premix_bwd(BF16, B, N, H, P, d, x, w, kw.get("dout", dout),
                                                kw.get("dx", dx), kw.get("dw", dw), kw.get("ws", ws),
                                                kw.get("wsz", wsz))
    assert cb() == OK
    assert cb(wsz=wsz - 1) == WORKSPACE and cb(ws=0) == WORKSPACE
    assert cb(dx=dout) == ALIAS and cb(dw=dx + 16) == ALIAS


def test_size_limits(lib):
    """A (b, h) slice spans at most 2^31 elements (the kernels address rows
    inside a slice with 32-bit offsets); whole tensors may be larger."""
    far = [(1 << 44) + i * (1 << 41) for i in range(5)]        # 2 TiB apart: no overlap
    def chk(B, Nq, Nk, d, mask=0, window=0):
        q, k, v, o, lse = far
        return lib.attn_check_fwd(BF16, B, 1, Nq, Nk, d, 0.125, mask, window, q, k, v, o, lse)
    assert chk(1, 1 << 25, 1 << 25, 64) == OK                 # Nq * d = 2^31 exactly
    assert chk(1, (1 << 25) + 1, 64, 64) == INVALID           # query slice past 2^31
    assert chk(1, 64, (1 << 25) + 1, 64) == INVALID           # key slice past 2^31
    assert chk(1, (1 << 24) + 16, 64, 128) == INVALID         # d = 128: 2^24 rows is the bound
    assert chk(4, 1 << 24, 1 << 24, 64, mask=2, window=64) == OK   # 2^32 elements per tensor
    assert chk(1, (1 << 30) + 1, 64, 64) == INVALID           # row count past 2^30


def test_noalloc_rejects_rows_beyond_its_scratch(lib):
    """attn_bwd_noalloc keeps the row sums in a 16 MiB array of its own: a
    call needing more (4 B H Nq bytes, rounded up to 256) is refused with
    ATTN_ERR_WORKSPACE before any pointer or device is touched; geometry
    errors come first, as in attn_bwd."""
    f = lib.attn_bwd_noalloc
    args = lambda B, H, Nq, d=128: (BF16, B, H, Nq, Nq, d, 0.125, MASK["causal"], 0) + (None,) * 9 + (None,)
    assert f(*args(1, 1, 4 * 1024 * 1024 + 1)) == WORKSPACE
    assert f(*args(2, 8, 300000)) == WORKSPACE
    assert f(*args(1, 1, 1000, d=80)) == UNSUPPORTED
    assert f(*args(0, 1, 1000)) == INVALID
    # the largest accepted row count needs exactly the scratch size
    assert lib.attn_bwd_workspace_size(1, 1, 4 * 1024 * 1024) == binding.NOALLOC_SCRATCH_BYTES
    assert lib.attn_bwd_workspace_size(1, 1, 4 * 1024 * 1024 + 1) > binding.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_is_not_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.lib_path()],
                         capture_output=True, text=True).stdout
    assert not [l for l in out.splitlines() if "scratch" in l]
