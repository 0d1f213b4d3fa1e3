"""Strided tensors at the C ABI, on the CPU: attn_layouts_contiguous, and
the validation of attn_check_fwd_strided / attn_check_bwd_strided (layout
rules, alignment, window maps, and the exact overlap test for interleaved
views of one buffer, against a brute-force byte-set comparison)."""
import ctypes
import itertools
import random

import pytest

from head_attention_attn_amd import binding
from head_attention_attn_amd.binding import Layout, Layouts

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, ALIAS = range(6)
BF16, FP32 = 0, 1
NONE, CAUSAL, SLIDING, BLOCK = range(4)
BASE = 1 << 40


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def contiguous(lib, B, H, Nq, Nk, d, mask=NONE, window=0):
    L = Layouts()
    assert lib.attn_layouts_contiguous(B, H, Nq, Nk, d, mask, window, ctypes.byref(L)) == OK
    return L


def check_fwd(lib, L, B, H, Nq, Nk, d, ptr, mask=NONE, window=0, dtype=BF16):
    """ptr: dict of byte addresses for q, k, v, o, lse."""
    return lib.attn_check_fwd_strided(dtype, B, H, Nq, Nk, d, 0.1, mask, window, ptr["q"], ptr["k"],
                                      ptr["v"], ptr["o"], ptr["lse"], ctypes.byref(L))


def check_bwd(lib, L, B, H, Nq, Nk, d, ptr, mask=NONE, window=0, dtype=BF16):
    ws = lib.attn_bwd_workspace_size(B, H, Nq)
    return lib.attn_check_bwd_strided(dtype, B, H, Nq, Nk, d, 0.1, mask, window, ptr["q"], ptr["k"],
                                      ptr["v"], ptr["o"], ptr["lse"], ptr["dout"], ptr["dq"],
                                      ptr["dk"], ptr["dv"], ptr["ws"], ws, ctypes.byref(L))


def far_ptrs():
    names = ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "ws"]
    return {n: BASE + i * (1 << 36) for i, n in enumerate(names)}


def test_contiguous_layouts(lib):
    L = contiguous(lib, 2, 3, 40, 96, 64, BLOCK, 24)       # 4 windows, 10 query rows each
    assert (L.q.batch, L.q.head, L.q.window, L.q.token) == (3 * 40 * 64, 40 * 64, 10 * 64, 64)
    assert (L.k.batch, L.k.head, L.k.window, L.k.token) == (3 * 96 * 64, 96 * 64, 24 * 64, 64)
    for n in ("o", "dout", "dq"):
        assert (getattr(L, n).batch, getattr(L, n).window) == (L.q.batch, L.q.window)
    for n in ("v", "dk", "dv"):
        assert (getattr(L, n).head, getattr(L, n).window) == (L.k.head, L.k.window)
    L = contiguous(lib, 1, 1, 7, 9, 96)
    assert (L.q.window, L.k.window) == (7 * 96, 9 * 96)
    assert lib.attn_layouts_contiguous(1, 1, 8, 8, 64, BLOCK, 3, ctypes.byref(L)) == INVALID
    assert lib.attn_layouts_contiguous(1, 1, 8, 8, 64, NONE, 0, None) == INVALID


def test_contiguous_layouts_equal_the_contiguous_entry_points(lib):
    """The strided check with the contiguous layouts (or NULL) returns what
    the contiguous check returns, including for aliasing pointers."""
    B, H, N, d = 2, 3, 100, 64
    L = contiguous(lib, B, H, N, N, d)
    p = far_ptrs()
    assert check_fwd(lib, L, B, H, N, N, d, p) == OK
    p2 = dict(p, o=p["q"] + 64)
    want = lib.attn_check_fwd(BF16, B, H, N, N, d, 0.1, 0, 0, p2["q"], p2["k"], p2["v"], p2["o"],
                              p2["lse"])
    assert want == ALIAS and check_fwd(lib, L, B, H, N, N, d, p2) == ALIAS
    assert lib.attn_check_fwd_strided(BF16, B, H, N, N, d, 0.1, 0, 0, p2["q"], p2["k"], p2["v"],
                                      p2["o"], p2["lse"], None) == ALIAS


def hiera_layouts(B, nw, T, Tq, H, D):
    """Hiera's token order: qkv viewed as (B, T, nw, 3, H, D), token
    n = t * nw + w; pooled Q (Tq rows per window) and O in (B, Tq, nw, H, D);
    dq, dk, dv interleaved like q, k, v (dq in its own (B, Tq, nw, H, D))."""
    row = 3 * H * D
    kv = Layout(T * nw * row, D, row, nw * row)
    qo = Layout(Tq * nw * H * D, D, H * D, nw * H * D)
    L = Layouts()
    for n in ("k", "v", "dk", "dv"):
        setattr(L, n, kv)
    for n in ("q", "o", "dout", "dq"):
        setattr(L, n, qo)
    return L


def test_hiera_token_order_is_accepted(lib):
    """K and V read in place from one qkv buffer (offsets H*D, 2*H*D), Q, O,
    dO, dQ in their own pooled buffers, dK and dV written into one dkv-style
    buffer with the qkv strides."""
    B, nw, T, Tq, H, D = 2, 49, 64, 16, 2, 96
    L = hiera_layouts(B, nw, T, Tq, H, D)
    qkv, dqkv = BASE + 16 * (1 << 36), BASE + 20 * (1 << 36)
    p = far_ptrs()
    p.update(k=qkv + H * D * 2, v=qkv + 2 * H * D * 2, dk=dqkv + H * D * 2, dv=dqkv + 2 * H * D * 2)
    assert check_fwd(lib, L, B, H, nw * Tq, nw * T, D, p, BLOCK, T) == OK
    assert check_bwd(lib, L, B, H, nw * Tq, nw * T, D, p, BLOCK, T) == OK
    # dK at V's offset in the dkv buffer collides with dV
    assert check_bwd(lib, L, B, H, nw * Tq, nw * T, D, dict(p, dk=p["dv"]), BLOCK, T) == ALIAS
    # dV written over the qkv input buffer's V slots
    assert check_bwd(lib, L, B, H, nw * Tq, nw * T, D, dict(p, dv=p["v"]), BLOCK, T) == ALIAS
    # dV into the qkv buffer's (unused by this call) Q slots: disjoint from k and v
    assert check_bwd(lib, L, B, H, nw * Tq, nw * T, D, dict(p, dv=qkv), BLOCK, T) == OK


def test_layout_rules(lib):
    B, H, N, d = 2, 2, 64, 64
    p = far_ptrs()
    base = contiguous(lib, B, H, N, N, d)

    def with_q(**kw):
        L = Layouts.from_buffer_copy(base)
        lay = Layout(L.q.batch, L.q.head, L.q.window, L.q.token)
        for k, v in kw.items():
            setattr(lay, k, v)
        L.q = lay
        return check_fwd(lib, L, B, H, N, N, d, p)

    assert with_q() == OK
    assert with_q(token=32) == INVALID               # rows overlap (token stride < d)
    assert with_q(head=64 * 63) == INVALID           # heads overlap the slice's rows
    assert with_q(token=-64) == INVALID
    assert with_q(batch=1 << 49) == INVALID          # stride above 2^48
    assert with_q(token=(1 << 26), head=(1 << 32), batch=(1 << 33)) == INVALID  # slice > 2^31
    assert with_q(token=(1 << 25), head=(1 << 31), batch=(1 << 32)) == OK       # just below
    assert with_q(token=72, head=72 * 64, batch=72 * 128) == OK        # padded rows (144 bytes)
    assert with_q(token=68, head=68 * 64, batch=68 * 128) == MISALIGNED  # 136-byte rows
    # B = 1: the batch stride is never used
    L1 = contiguous(lib, 1, H, N, N, d)
    L1.q = Layout(3, L1.q.head, L1.q.window, L1.q.token)
    assert check_fwd(lib, L1, 1, H, N, N, d, p) == OK


def test_interleaved_windows_need_power_of_two_lengths(lib):
    """Windows that do not follow each other at the token stride: T must be
    a power of two (the kernels split the token index with a shift)."""
    p = far_ptrs()
    for T, want in ((16, OK), (64, OK), (24, UNSUPPORTED), (1, OK)):
        nw, d = 6, 64
        row = 3 * d
        L = contiguous(lib, 1, 1, nw * T, nw * T, d, BLOCK, T)
        lay = Layout(0, 0, row, nw * row)
        L.q = L.k = L.v = lay
        ptr = dict(p, k=p["q"] + 2 * d, v=p["q"] + 4 * d)
        assert check_fwd(lib, L, 1, 1, nw * T, nw * T, d, ptr, BLOCK, T) == want, T
    # a uniform layout (windows at the token stride) of any length is fine
    L = contiguous(lib, 1, 1, 6 * 24, 6 * 24, 64, BLOCK, 24)
    assert check_fwd(lib, L, 1, 1, 144, 144, 64, p, BLOCK, 24) == OK


def byte_set(base, lay, B, H, nwin, T, d, es):
    out = set()
    for b, h, w, t in itertools.product(range(B), range(H), range(nwin), range(T)):
        r = base + es * (b * lay.batch + h * lay.head + w * lay.window + t * lay.token)
        out.update(range(r, r + es * d))
    return out


def dims_of(lay, B, H, nwin, T):
    return sorted((s, n) for s, n in ((lay.batch, B), (lay.head, H), (lay.window, nwin),
                                      (lay.token, T)) if n > 1)


def nested(lay, B, H, nwin, T, d):
    dims = dims_of(lay, B, H, nwin, T)
    need = d
    for s, n in dims:
        if s < need:
            return False
        need = s * n
    return True


def test_exact_overlap_against_brute_force(lib):
    """Random nested layouts of small tensors: o against q.  Same strides and
    extents: ALIAS exactly when the byte sets meet; otherwise ALIAS when the
    address ranges meet (the documented conservative rule)."""
    rng = random.Random(5)
    d, es = 64, 2
    seen = {OK: 0, ALIAS: 0}
    for trial in range(300):
        B, H, nw, T = rng.choice([1, 2]), rng.choice([1, 2, 3]), rng.choice([1, 2, 4]), rng.choice([1, 2, 4])
        dims = [(n, rng.choice([1, 2, 3])) for n in ("token", "head", "window", "batch")]
        rng.shuffle(dims)
        lay = Layout()
        stride = d
        ext = {"batch": B, "head": H, "window": nw, "token": T}
        for name, gap in dims:
            setattr(lay, name, stride * gap if ext[name] > 1 else 0)
            stride = stride * gap * max(ext[name], 1)
        same = rng.random() < 0.8
        lay_o = lay if same else Layout(lay.batch, lay.head, lay.window, lay.token + 8 * (T > 1))
        if not nested(lay_o, B, H, nw, T, d):
            continue
        L = contiguous(lib, B, H, nw * T, nw * T, d, BLOCK, T)
        L.q = lay
        L.o = lay_o
        shift = 16 * rng.randrange(-320, 320)
        p = far_ptrs()
        p["o"] = p["q"] + shift
        got = check_fwd(lib, L, B, H, nw * T, nw * T, d, p, BLOCK, T)
        sq = byte_set(p["q"], lay, B, H, nw, T, d, es)
        so = byte_set(p["o"], lay_o, B, H, nw, T, d, es)
        if dims_of(lay, B, H, nw, T) == dims_of(lay_o, B, H, nw, T):
            want = ALIAS if sq & so else OK
        else:
            want = ALIAS if (min(so) <= max(sq) and min(sq) <= max(so)) else OK
        assert got == want, (trial, B, H, nw, T, shift, [getattr(lay, n) for n in ext])
        seen[got] += 1
    assert seen[OK] > 30 and seen[ALIAS] > 30
