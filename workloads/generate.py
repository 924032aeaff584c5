"""Seeded input draws: i.i.d. N(0, 1) fp32 rounded to bf16 (round-to-nearest-even).

Draw order is fixed: Q, K, V, then dO, all from one CPU torch generator seeded
with the workload's seed, each of shape [B, S, H, D] (H = heads_kv for K and V).
The ring-step order of key/value chunks is a seeded permutation from numpy's
default generator.
"""
from __future__ import annotations

import numpy as np
import torch


def make_inputs(batch, seqlen, heads_q, heads_kv, head_dim, *, seed=0, with_dout=False,
                q_scale=1.0, seqlen_k=None):
    """Return bf16 CPU tensors (q, k, v[, dout]) in [B, S, H, D] layout.

    q_scale multiplies Q before rounding (a value > 1 gives a peaked softmax).
    """
    sk = seqlen if seqlen_k is None else seqlen_k
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn(batch, seqlen, heads_q, head_dim, generator=g, dtype=torch.float32)
    if q_scale != 1.0:
        q = q * q_scale
    q = q.to(torch.bfloat16)
    k = torch.randn(batch, sk, heads_kv, head_dim, generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(batch, sk, heads_kv, head_dim, generator=g, dtype=torch.float32).to(torch.bfloat16)
    if not with_dout:
        return q, k, v
    do = torch.randn(batch, seqlen, heads_q, head_dim, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, do


def chunk_order(n_chunks, seed=0):
    """Seeded random order in which the ring steps visit the key/value chunks."""
    return [int(c) for c in np.random.default_rng(seed).permutation(n_chunks)]


def chunk_bounds(seqlen_k, n_chunks):
    """[start, end) of each chunk; equal chunks of ceil(S/n), the last one possibly shorter."""
    c = -(-seqlen_k // n_chunks)
    return [(i * c, min((i + 1) * c, seqlen_k)) for i in range(n_chunks) if i * c < seqlen_k]


def make_ffn_inputs(rows, d_model, d_ff, *, seed=0):
    """Return bf16 CPU tensors (x, w1, w3, w2) for the blockwise feedforward.

    x [rows, d_model] ~ N(0, 1) (activations); the weights are random in the layout of a linear
    layer ([out, in]) with the usual fan-in scaling, w1, w3 [d_ff, d_model] ~ N(0, 1/d_model) and
    w2 [d_model, d_ff] ~ N(0, 1/d_ff), so every pre-activation is O(1).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(rows, d_model, generator=g, dtype=torch.float32).to(torch.bfloat16)
    w1 = (torch.randn(d_ff, d_model, generator=g, dtype=torch.float32) / d_model ** 0.5).to(torch.bfloat16)
    w3 = (torch.randn(d_ff, d_model, generator=g, dtype=torch.float32) / d_model ** 0.5).to(torch.bfloat16)
    w2 = (torch.randn(d_model, d_ff, generator=g, dtype=torch.float32) / d_ff ** 0.5).to(torch.bfloat16)
    return x, w1, w3, w2
