"""MI355X-native fused multi-head attention (forward + backward).

The compute path is the C-ABI library ``libattn.so`` (hand-written gfx950 HIP
kernels); ``fwd`` and ``bwd`` here only marshal torch device tensors into its
entry points.  The library is loaded on first use and its absence is an error:
there is no fallback path.
"""
from .binding import fwd, bwd, lib_path, load_library, AttnError, MASK_CODES, premix_bwd
from .autograd import (FusedAttention, FusedAttentionFunction, PremixFunction, fused_attention,
                       iha_attention, premix)

__all__ = ["fwd", "bwd", "lib_path", "load_library", "AttnError", "MASK_CODES",
           "FusedAttention", "FusedAttentionFunction", "fused_attention", "PremixFunction",
           "premix", "premix_bwd", "iha_attention"]
