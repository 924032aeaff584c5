"""S2-Attn (LongLoRA summary, Summary): grouped causal attention, half of the heads shifted.

The roll is not materialised: the library's tile scheduler maps rolled
positions to original rows, so inputs and outputs stay at original positions.
"""
from __future__ import annotations

import torch

from . import _lib


def s2_forward(q, k, v, group, shift_head0=None, *, scale=None, o_dtype=torch.bfloat16, stream=None):
    """Returns (o [B,S,Hq,D] of o_dtype, lse fp32 [B,Hq,S]); heads [shift_head0, Hq) are shifted."""
    b, s, hq, d = q.shape
    shift_head0 = hq // 2 if shift_head0 is None else shift_head0
    o = torch.empty(b, s, hq, d, device=q.device, dtype=o_dtype)
    lse = torch.empty(b, hq, s, device=q.device, dtype=torch.float32)
    _lib.s2attn_fwd(q, k, v, o, lse, group=group, shift_head0=shift_head0, scale=scale, stream=stream)
    return o, lse


def s2_backward(q, k, v, o, dout, lse, group, shift_head0=None, *, scale=None,
                dkv_dtype=torch.bfloat16, stream=None):
    """Returns (dq bf16, dk, dv) of <dout, O> under the S2 mask."""
    b, s, hq, d = q.shape
    shift_head0 = hq // 2 if shift_head0 is None else shift_head0
    delta = torch.empty(b, hq, s, device=q.device, dtype=torch.float32)
    dq_acc = torch.zeros(b, s, hq, d, device=q.device, dtype=torch.float32)
    dq = torch.empty(b, s, hq, d, device=q.device, dtype=torch.bfloat16)
    dk = torch.empty(k.shape, device=k.device, dtype=dkv_dtype)
    dv = torch.empty(v.shape, device=v.device, dtype=dkv_dtype)
    _lib.s2attn_bwd(q, k, v, o, dout, lse, delta, dq_acc, dk, dv, group=group, shift_head0=shift_head0,
                    dq_final=dq, flags=_lib.BA_BWD_COMPUTE_DELTA | _lib.BA_BWD_FINALIZE_DQ,
                    scale=scale, stream=stream)
    return dq, dk, dv
