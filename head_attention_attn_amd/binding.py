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
DTYPE_CODES = {torch.bfloat16: 0, torch.float32: 1}

_lib = None


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
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _geometry(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if q.dtype not in DTYPE_CODES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype bfloat16 or float32")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
    return B, H, Nq, k.shape[2], d


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def fwd(q, k, v, mask: str = "none", window: int = 0, scale=None, out=None, lse=None):
    """O, lse = attention(q, k, v).  Returns (o [B,H,Nq,d] in q.dtype,
    lse [B,H,Nq] float32)."""
    lib = load_library()
    B, H, Nq, Nk, d = _geometry(q, k, v)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    st = lib.attn_fwd(DTYPE_CODES[q.dtype], B, H, Nq, Nk, d, _scale(scale, d),
                      MASK_CODES[mask], int(window), q.data_ptr(), k.data_ptr(),
                      v.data_ptr(), o.data_ptr(), lse.data_ptr(), _stream(q))
    if st != 0:
        raise AttnError(st, "attn_fwd")
    return o, lse


def bwd_fused(q, k, v, mask: str = "none", window: int = 0) -> bool:
    """True when ``bwd`` runs as one fused kernel for these tensors (then
    ``passes`` must be PASS_ALL)."""
    B, H, Nq, Nk, d = _geometry(q, k, v)
    return load_library().attn_bwd_fused(DTYPE_CODES[q.dtype], B, H, Nq, Nk, d,
                                         MASK_CODES[mask], int(window)) == 1


def workspace_bytes(B: int, H: int, Nq: int) -> int:
    """Minimum backward workspace (row sums only)."""
    return int(load_library().attn_bwd_workspace_size(B, H, Nq))


def workspace_bytes_ds(q, k, mask: str = "none", window: int = 0) -> int:
    """Backward workspace with which the dQ pass reads dS kept by the dK/dV
    pass (``attn_bwd_workspace_size_ds``); equals ``workspace_bytes`` where
    that path does not apply."""
    B, H, Nq, d = q.shape
    return int(load_library().attn_bwd_workspace_size_ds(
        DTYPE_CODES[q.dtype], B, H, Nq, k.shape[2], d, MASK_CODES[mask], int(window)))


PASS_ROWSUM, PASS_DKDV, PASS_DQ, PASS_ALL = 1, 2, 4, 7


def bwd(q, k, v, o, lse, do, mask: str = "none", window: int = 0, scale=None,
        workspace=None, dq=None, dk=None, dv=None, passes: int = PASS_ALL,
        keep_ds: bool = True):
    """dQ, dK, dV of attention given dO.  Returns tensors shaped like q, k, v.
    ``passes`` (a set of PASS_* bits) restricts the call to some of the
    backward passes (``attn_bwd_passes``); the default runs all three.  When
    no workspace is given one is allocated: with ``keep_ds`` large enough
    for the dQ pass to read dS kept by the dK/dV pass, else the minimum."""
    lib = load_library()
    B, H, Nq, Nk, d = _geometry(q, k, v)
    if o.shape != q.shape or do.shape != q.shape or lse.shape != (B, H, Nq):
        raise ValueError("o/do must match q and lse must be [B, H, Nq]")
    ws_need = workspace_bytes_ds(q, k, mask, window) if keep_ds else workspace_bytes(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    st = lib.attn_bwd_passes(int(passes), DTYPE_CODES[q.dtype], B, H, Nq, Nk, d, _scale(scale, d),
                      MASK_CODES[mask], int(window), q.data_ptr(), k.data_ptr(),
                      v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                      workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise AttnError(st, "attn_bwd_passes")
    return dq, dk, dv
