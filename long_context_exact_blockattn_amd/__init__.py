"""Exact blockwise causal attention for MI355X (gfx950).

The compute lives in libblockattn.so (HIP kernels behind a C ABI, declared in
include/blockattn.h).  This package is its thin Python binding (_lib) plus the
sequential ring-step and S2 drivers, which only issue library calls.
"""
from . import _lib
from ._lib import (BA_ACCUMULATE, BA_FINAL_REACHED_ONLY, BA_BWD_COMPUTE_DELTA, BA_BWD_FINALIZE_DQ, BA_OVERWRITE,
                   BlockAttnError, blockattn_bwd, blockattn_bwd_noalloc, blockattn_fwd, lse_merge,
                   s2attn_bwd, s2attn_fwd, bpt_ffn, status_string, ulysses_pack, ulysses_unpack)
from .ring import ring_backward, ring_forward, ring_forward_staged
from .s2 import s2_backward, s2_forward

__all__ = [
    "BA_ACCUMULATE", "BA_FINAL_REACHED_ONLY", "BA_BWD_COMPUTE_DELTA", "BA_BWD_FINALIZE_DQ", "BA_OVERWRITE", "BlockAttnError",
    "blockattn_bwd", "blockattn_bwd_noalloc", "blockattn_fwd", "lse_merge", "s2attn_bwd", "s2attn_fwd", "status_string",
    "ring_backward", "ring_forward", "ring_forward_staged", "s2_backward", "s2_forward",
    "ulysses_pack", "ulysses_unpack", "bpt_ffn",
]
