"""ctypes binding of libattn (include/attn.h).

Argument marshalling only: shapes and dtypes are read off torch tensors, the
tensors' device pointers and torch's current HIP stream are handed to the C
entry points, and a nonzero status becomes an ``AttnError``.  All arithmetic
runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))

MASK_CODES = {"none": 0, "causal": 1, "sliding": 2, "block": 3}
DTYPE_CODES = {torch.bfloat16: 0, torch.float32: 1, torch.float16: 2}

_lib = None


class Layout(ctypes.Structure):
    """``attn_layout``: element strides of one tensor's rows."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64),
                ("window", ctypes.c_int64), ("token", ctypes.c_int64)]


class Layouts(ctypes.Structure):
    """``attn_layouts``: the layouts of every tensor argument."""
    _fields_ = [(n, Layout) for n in ("q", "k", "v", "o", "dout", "dq", "dk", "dv")]


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def lib_path() -> str:
    return os.path.join(_HERE, "libattn.so")


def load_library():
    """Load libattn.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    i64, vp, fp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.attn_fwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_float,
                             ctypes.c_int, i64, vp, vp, vp, vp, fp, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_float,
                             ctypes.c_int, i64, vp, vp, vp, vp, fp, vp, vp, vp, vp,
                             vp, ctypes.c_size_t, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_passes.argtypes = [ctypes.c_int] + lib.attn_bwd.argtypes
    lib.attn_bwd_passes.restype = ctypes.c_int
    lib.attn_bwd_fused.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_int, i64]
    lib.attn_bwd_fused.restype = ctypes.c_int
    lib.attn_bwd_workspace_size.argtypes = [i64, i64, i64]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_size_ds.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64,
                                               ctypes.c_int, i64]
    lib.attn_bwd_workspace_size_ds.restype = ctypes.c_size_t
    lib.attn_check_fwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_float,
                                   ctypes.c_int, i64, vp, vp, vp, vp, fp]
    lib.attn_check_fwd.restype = ctypes.c_int
    lib.attn_check_bwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_float,
                                   ctypes.c_int, i64, vp, vp, vp, vp, fp, vp, vp, vp, vp,
                                   vp, ctypes.c_size_t]
    lib.attn_check_bwd.restype = ctypes.c_int
    lp = ctypes.POINTER(Layouts)
    lib.attn_fwd_strided.argtypes = lib.attn_fwd.argtypes[:-1] + [lp, vp]
    lib.attn_fwd_strided.restype = ctypes.c_int
    lib.attn_bwd_strided.argtypes = [ctypes.c_int] + lib.attn_bwd.argtypes[:-1] + [lp, vp]
    lib.attn_bwd_strided.restype = ctypes.c_int
    lib.attn_check_fwd_strided.argtypes = lib.attn_check_fwd.argtypes + [lp]
    lib.attn_check_fwd_strided.restype = ctypes.c_int
    lib.attn_check_bwd_strided.argtypes = lib.attn_check_bwd.argtypes + [lp]
    lib.attn_check_bwd_strided.restype = ctypes.c_int
    lib.attn_layouts_contiguous.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, i64, lp]
    lib.attn_layouts_contiguous.restype = ctypes.c_int
    lib.attn_premix_fwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, vp, vp, vp, vp]
    lib.attn_premix_fwd.restype = ctypes.c_int
    lib.attn_premix_bwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, vp, vp, vp, vp, fp, vp,
                                    ctypes.c_size_t, vp]
    lib.attn_premix_bwd.restype = ctypes.c_int
    lib.attn_premix_bwd_workspace_size.argtypes = [i64, i64, i64, i64]
    lib.attn_premix_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_check_premix_fwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, vp, vp, vp]
    lib.attn_check_premix_fwd.restype = ctypes.c_int
    lib.attn_check_premix_bwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, vp, vp, vp, vp, fp,
                                          vp, ctypes.c_size_t]
    lib.attn_check_premix_bwd.restype = ctypes.c_int
    lib.attn_bwd_noalloc.argtypes = lib.attn_bwd.argtypes[:-3] + [vp]
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _rows(t, name):
    """(B, H, n, T, d, Layout) of a [B, H, N, d] tensor (any row strides) or
    of a window-split [B, nw, H, T, d] one (block mask: window w, position t
    is token w * T + t); the d values of a row must be contiguous."""
    if t.dim() == 4:
        B, H, n, d = t.shape
        sb, sh, st, sd = t.stride()
        lay, T = Layout(sb, sh, 0, st), n
    elif t.dim() == 5:
        B, nw, H, T, d = t.shape
        sb, sw, sh, st, sd = t.stride()
        lay, n = Layout(sb, sh, sw, st), nw * T
    else:
        raise ValueError(f"{name} must be [B, H, N, d] or [B, nw, H, T, d]")
    if d > 1 and sd != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return B, H, n, T, d, lay


def rows_usable(t) -> bool:
    """Whether ``t`` can be passed as it is: contiguous rows, a 16-byte
    aligned base, and every stride of a dimension of size > 1 a positive
    multiple of 16 bytes (the library checks the rest)."""
    if t.stride(-1) != 1 or t.data_ptr() % 16:
        return False
    per16 = 16 // t.element_size()
    return all(st > 0 and st % per16 == 0 for n, st in zip(t.shape[:-1], t.stride()[:-1]) if n > 1)


def _geometry(q, k, v, mask=None, window=None):
    """Shapes, mask and window of a call: (B, H, Nq, Nk, d, mask, window).
    Window-split (5-D) tensors mean the block mask with window = T of k."""
    if not (q.dim() == k.dim() == v.dim()):
        raise ValueError("q, k, v must all be 4-D or all 5-D")
    Bq, Hq, Nq, Tq, d, _ = _rows(q, "q")
    B, H, Nk, Tk, dk, _ = _rows(k, "k")
    if (Bq, Hq, dk) != (B, H, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if q.dtype not in DTYPE_CODES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bfloat16, float16 or float32")
    if q.dim() == 5:
        if q.shape[1] != k.shape[1]:
            raise ValueError("q and k must have the same number of windows")
        if mask not in (None, "block") or window not in (None, 0, Tk):
            raise ValueError("window-split tensors take the block mask with window = T of k")
        mask, window = "block", Tk
    return B, H, Nq, Nk, d, mask or "none", int(window or 0)


def _is_plain(*ts):
    return all(t.dim() == 4 and t.is_contiguous() for t in ts)


def _empty_rows(like):
    """An output shaped like ``like``: contiguous for 4-D; for 5-D
    [B, nw, H, T, d], stored in token order (B, T, nw, H, d) -- position-major
    with the window index fastest, the order Hiera's output projection reads."""
    if like.dim() == 4:
        return torch.empty(like.shape, dtype=like.dtype, device=like.device)
    B, nw, H, T, d = like.shape
    return torch.empty((B, T, nw, H, d), dtype=like.dtype, device=like.device).permute(0, 2, 3, 1, 4)


_Q_SIDE = ("q", "o", "dout", "dq")


def _layouts(Nq, Nk, mask, window, **ts):
    """attn_layouts of the named tensors.  A [B, H, N, d] tensor's windows
    (block mask) follow each other at its token stride."""
    L = Layouts()
    for name, t in ts.items():
        lay = _rows(t, name)[5]
        if t.dim() == 4:
            n = Nq if name in _Q_SIDE else Nk
            T = n if mask != "block" else (window if name not in _Q_SIDE else Nq // (Nk // window))
            lay.window = T * lay.token
        setattr(L, name, lay)
    return L


def _mask_args(q, mask, window):
    """The caller's mask and window as _geometry takes them: for window-split
    tensors the defaults ("none", 0) mean "from the tensors"."""
    if q.dim() == 5:
        return (None if mask == "none" else mask), (None if not window else window)
    return mask, window


def _check_out(t, like, name):
    """A caller-provided output: on like's device, in like's dtype and shape
    (its rows may be strided like the inputs')."""
    if not isinstance(t, torch.Tensor) or t.device != like.device or t.dtype != like.dtype \
            or tuple(t.shape) != tuple(like.shape):
        raise ValueError(f"{name} must be a {like.dtype} tensor shaped {tuple(like.shape)} "
                         f"on {like.device}")
    return t


def _check_lse(t, B, H, Nq, device):
    """lse: a contiguous float32 [B, H, Nq] device tensor (the library writes
    B * H * Nq floats at its base)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != device \
            or tuple(t.shape) != (B, H, Nq) or not t.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 tensor [{B}, {H}, {Nq}] on {device}")
    return t


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def fwd(q, k, v, mask: str = "none", window: int = 0, scale=None, out=None, lse=None):
    """O, lse = attention(q, k, v).  q, k, v: [B, H, N, d] with any row
    strides (contiguous ones take ``attn_fwd``, others ``attn_fwd_strided``),
    or window-split [B, nw, H, T, d] views (block mask, window T).  Returns
    (o shaped like q, in q.dtype; lse [B, H, Nq] float32)."""
    lib = load_library()
    B, H, Nq, Nk, d, mask, window = _geometry(q, k, v, *_mask_args(q, mask, window))
    o = _empty_rows(q) if out is None else _check_out(out, q, "out")
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None \
        else _check_lse(lse, B, H, Nq, q.device)
    args = (DTYPE_CODES[q.dtype], B, H, Nq, Nk, d, _scale(scale, d), MASK_CODES[mask], window,
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    if _is_plain(q, k, v, o):
        st = lib.attn_fwd(*args, _stream(q))
    else:
        L = _layouts(Nq, Nk, mask, window, q=q, k=k, v=v, o=o)
        st = lib.attn_fwd_strided(*args, ctypes.byref(L), _stream(q))
    if st != 0:
        raise AttnError(st, "attn_fwd")
    return o, lse


def bwd_fused(q, k, v, mask: str = "none", window: int = 0) -> int:
    """Nonzero when ``bwd`` runs as one fused kernel for these tensors:
    FUSED_LOCAL (block-local windows; ``passes`` must then be PASS_ALL) or
    FUSED_SHORT (every key of a (b, h) in one workgroup; a partial ``passes``
    set runs the general passes); 0 otherwise."""
    B, H, Nq, Nk, d, mask, window = _geometry(q, k, v, *_mask_args(q, mask, window))
    return int(load_library().attn_bwd_fused(DTYPE_CODES[q.dtype], B, H, Nq, Nk, d,
                                             MASK_CODES[mask], window))


FUSED_LOCAL, FUSED_SHORT = 1, 2


def workspace_bytes(B: int, H: int, Nq: int) -> int:
    """Minimum backward workspace (row sums only)."""
    return int(load_library().attn_bwd_workspace_size(B, H, Nq))


def workspace_bytes_ds(q, k, mask: str = "none", window: int = 0) -> int:
    """Backward workspace with which the dQ pass reads dS kept by the dK/dV
    pass (``attn_bwd_workspace_size_ds``); equals ``workspace_bytes`` where
    that path does not apply."""
    B, H, Nq, Nk, d, mask, window = _geometry(q, k, k, *_mask_args(q, mask, window))
    return int(load_library().attn_bwd_workspace_size_ds(
        DTYPE_CODES[q.dtype], B, H, Nq, Nk, d, MASK_CODES[mask], window))


PASS_ROWSUM, PASS_DKDV, PASS_DQ, PASS_ALL = 1, 2, 4, 7


def bwd(q, k, v, o, lse, do, mask: str = "none", window: int = 0, scale=None,
        workspace=None, dq=None, dk=None, dv=None, passes: int = PASS_ALL,
        keep_ds: bool = True):
    """dQ, dK, dV of attention given dO.  Returns tensors shaped like q, k, v
    (any row strides, or window-split views, as for ``fwd``).
    ``passes`` (a set of PASS_* bits) restricts the call to some of the
    backward passes (``attn_bwd_passes``); the default runs all three.  When
    no workspace is given one is allocated: with ``keep_ds`` large enough
    for the dQ pass to read dS kept by the dK/dV pass, else the minimum."""
    lib = load_library()
    B, H, Nq, Nk, d, mask, window = _geometry(q, k, v, *_mask_args(q, mask, window))
    _check_out(o, q, "o")
    _check_out(do, q, "do")
    _check_lse(lse, B, H, Nq, q.device)
    ws_need = workspace_bytes_ds(q, k, mask, window) if keep_ds else workspace_bytes(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    dq = _empty_rows(q) if dq is None else _check_out(dq, q, "dq")
    dk = _empty_rows(k) if dk is None else _check_out(dk, k, "dk")
    dv = _empty_rows(v) if dv is None else _check_out(dv, v, "dv")
    if workspace is not None and (workspace.device != q.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    args = (int(passes), DTYPE_CODES[q.dtype], B, H, Nq, Nk, d, _scale(scale, d),
            MASK_CODES[mask], window, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
            lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size())
    if _is_plain(q, k, v, o, do, dq, dk, dv):
        st = lib.attn_bwd_passes(*args, _stream(q))
    else:
        L = _layouts(Nq, Nk, mask, window, q=q, k=k, v=v, o=o, dout=do, dq=dq, dk=dk, dv=dv)
        st = lib.attn_bwd_strided(*args, ctypes.byref(L), _stream(q))
    if st != 0:
        raise AttnError(st, "attn_bwd_passes")
    return dq, dk, dv


# size of the library's scratch array for attn_bwd_noalloc (include/attn.h)
NOALLOC_SCRATCH_BYTES = 16 << 20


def bwd_noalloc(q, k, v, o, lse, do, mask: str = "none", window: int = 0, scale=None,
                dq=None, dk=None, dv=None):
    """``attn_bwd_noalloc``: the backward with the row sums in the library's
    own device scratch array, so the call itself allocates nothing (outputs
    given by the caller are written in place; missing ones are allocated
    here).  Contiguous [B, H, N, d] tensors only.  Raises AttnError
    (ATTN_ERR_WORKSPACE) when 4 B H Nq bytes exceed the scratch array."""
    lib = load_library()
    B, H, Nq, Nk, d, mask, window = _geometry(q, k, v, *_mask_args(q, mask, window))
    _check_out(o, q, "o")
    _check_out(do, q, "do")
    _check_lse(lse, B, H, Nq, q.device)
    dq = _empty_rows(q) if dq is None else _check_out(dq, q, "dq")
    dk = _empty_rows(k) if dk is None else _check_out(dk, k, "dk")
    dv = _empty_rows(v) if dv is None else _check_out(dv, v, "dv")
    if not _is_plain(q, k, v, o, do, dq, dk, dv):
        raise ValueError("attn_bwd_noalloc takes contiguous [B, H, N, d] tensors only")
    st = lib.attn_bwd_noalloc(DTYPE_CODES[q.dtype], B, H, Nq, Nk, d, _scale(scale, d),
                              MASK_CODES[mask], window, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), _stream(q))
    if st != 0:
        raise AttnError(st, f"attn_bwd_noalloc ({workspace_bytes(B, H, Nq)} bytes of row sums, "
                            f"scratch holds {NOALLOC_SCRATCH_BYTES})")
    return dq, dk, dv


# ------------------------------------------------------------ IHA premix

def _premix_shapes(x, w):
    if x.dim() != 4 or w.dim() != 3:
        raise ValueError("x must be [B, N, H, d] and w [H, P, H]")
    B, N, H, d = x.shape
    if w.shape[0] != H or w.shape[2] != H:
        raise ValueError(f"w{tuple(w.shape)} does not match H = {H}")
    if x.dtype not in DTYPE_CODES or w.dtype != x.dtype:
        raise ValueError("x and w must share a 16-bit dtype")
    for t in (x, w):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("premix tensors must be contiguous device tensors")
    return B, N, H, w.shape[1], d


def _check_contiguous(t, shape, dtype, device, name):
    if not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype \
            or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor {list(shape)} on {device}")


def premix_workspace_bytes(B: int, N: int, H: int, P: int) -> int:
    return int(load_library().attn_premix_bwd_workspace_size(B, N, H, P))


def premix(x, w, out=None):
    """IHA pseudo-tokens: out[b, h, n, p] = sum_s w[h, p, s] x[b, n, s]
    (``attn_premix_fwd``).  x [B, N, H, d], w [H, P, H] -> out
    [B, H, N, P, d]; ``out.view(B, H, N * P, d)`` is each head's pseudo-token
    sequence."""
    lib = load_library()
    B, N, H, P, d = _premix_shapes(x, w)
    if out is None:
        out = torch.empty((B, H, N, P, d), dtype=x.dtype, device=x.device)
    _check_contiguous(out, (B, H, N, P, d), x.dtype, x.device, "out")
    st = lib.attn_premix_fwd(DTYPE_CODES[x.dtype], B, N, H, P, d, x.data_ptr(), w.data_ptr(),
                             out.data_ptr(), _stream(x))
    if st != 0:
        raise AttnError(st, "attn_premix_fwd")
    return out


def premix_bwd(x, w, dout, dx=None, dw=None, workspace=None):
    """dx = w^T dout, dw = sum over (b, n, feature) of dout x^T
    (``attn_premix_bwd``); dw is float32."""
    lib = load_library()
    B, N, H, P, d = _premix_shapes(x, w)
    if tuple(dout.shape) != (B, H, N, P, d) or dout.dtype != x.dtype or not dout.is_contiguous():
        raise ValueError("dout must be a contiguous [B, H, N, P, d] tensor of x's dtype")
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty((H, P, H), dtype=torch.float32, device=x.device) if dw is None else dw
    _check_contiguous(dx, tuple(x.shape), x.dtype, x.device, "dx")
    _check_contiguous(dw, (H, P, H), torch.float32, x.device, "dw")
    if workspace is None:
        workspace = torch.empty(premix_workspace_bytes(B, N, H, P), dtype=torch.uint8,
                                device=x.device)
    st = lib.attn_premix_bwd(DTYPE_CODES[x.dtype], B, N, H, P, d, x.data_ptr(), w.data_ptr(),
                             dout.data_ptr(), dx.data_ptr(), dw.data_ptr(), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), _stream(x))
    if st != 0:
        raise AttnError(st, "attn_premix_bwd")
    return dx, dw
