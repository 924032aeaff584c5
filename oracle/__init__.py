"""CPU oracle for exact blockwise causal attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and this package imports
nothing from the product path.

Every value is computed in float64 from the plain definition of softmax
attention; see oracle/attention.py for the readings taken where the pages are
silent.
"""
from .attention import (
    NEG_INF,
    S2Spec,
    allowed_mask,
    attention_backward,
    backward_delta,
    cols_backward_dkdv,
    rows_backward_dq,
    attention_forward,
    default_scale,
    lse_merge,
    ring_attention_forward,
    rows_forward,
)

__all__ = [
    "NEG_INF",
    "S2Spec",
    "allowed_mask",
    "attention_backward",
    "backward_delta",
    "cols_backward_dkdv",
    "rows_backward_dq",
    "attention_forward",
    "default_scale",
    "lse_merge",
    "ring_attention_forward",
    "rows_forward",
]
from . import ulysses  # noqa: E402,F401  (layout permutes of Ulysses sequence parallelism)
from . import ffn  # noqa: E402,F401  (blockwise feedforward, SwiGLU)
