"""Seeded synthetic workloads shared by the oracle side and the HIP side.

This module holds only shapes and random-number draws: no attention arithmetic.
Both the CPU oracle and the GPU path consume the tensors built here, so they see
bit-identical bf16 inputs.

Workload shapes follow the attention shapes of the models the pages name
(Llama-2-7B, Llama-2-13B, a Llama-3-8B-style GQA layout), with i.i.d. N(0, 1)
values standing in for activations (the pages train on PG19 / RedPajama /
ShareGPT text with trained weights; none of that is used here).
"""
from .configs import CONFIGS, FFN_CONFIGS, FfnWorkload, Workload, get
from .generate import chunk_bounds, chunk_order, make_ffn_inputs, make_inputs

__all__ = ["CONFIGS", "FFN_CONFIGS", "FfnWorkload", "Workload", "get", "chunk_order", "make_inputs",
           "make_ffn_inputs", "chunk_bounds"]
