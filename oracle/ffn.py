"""Oracle of the blockwise feedforward (TEST INFRASTRUCTURE ONLY: imported by tests/ and bench.py's
CPU baseline, never by the library).

Ring Attention's hosts compute attention AND the feedforward for their query block, block by block
(Ring Attention summary, Summary; the blockwise parallel transformer it extends computes the
feedforward per block so that the full hidden activation of the sequence never exists, Key
points).  The pages do not print the feedforward; the models they train are LLaMA / Llama-2, whose
feedforward is SwiGLU:
    FFN(x) = (silu(x W1^T) * (x W3^T)) W2^T,   silu(z) = z / (1 + e^-z)
with x [rows, d_model], W1, W3 [d_ff, d_model], W2 [d_model, d_ff] (the [out, in] layout of a
linear layer).  Rows are independent, so any blocking of the rows gives the same result; the
oracle evaluates the plain definition in float64 on the bf16-rounded inputs.
"""
from __future__ import annotations

import numpy as np


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(x, w1, w3, w2):
    """The feedforward of every row of x, in float64."""
    x = np.asarray(x, dtype=np.float64)
    w1, w3, w2 = (np.asarray(w, dtype=np.float64) for w in (w1, w3, w2))
    return (silu(x @ w1.T) * (x @ w3.T)) @ w2.T


def swiglu_hidden(x, w1, w3):
    """The hidden activation silu(x W1^T) * (x W3^T) of every row, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return silu(x @ np.asarray(w1, dtype=np.float64).T) * (x @ np.asarray(w3, dtype=np.float64).T)
