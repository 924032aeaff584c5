"""The workload shapes used for parity tests and throughput measurement.

Each entry names what it is: the model whose attention shape it copies, the
sequence length, and how the key/value sequence is streamed (ring steps of
equal chunks whose partial (O, LSE) pairs are merged), or the S2 grouping.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    n_chunks: int = 1            # ring steps over the key/value sequence
    s2_group: Optional[int] = None   # S2-Attn group size (None: plain causal)
    s2_shift_head0: Optional[int] = None  # first shifted head
    backward: bool = False
    seed: int = 0
    description: str = ""

    @property
    def chunk_len(self) -> int:
        return -(-self.seqlen // self.n_chunks)

    def allowed_pairs_per_head(self) -> int:
        """Number of (query, key) pairs the mask allows, per (batch, head)."""
        s = self.seqlen
        if self.s2_group is None:
            return s * (s + 1) // 2
        g = self.s2_group
        return (s // g) * g * (g + 1) // 2

    def fwd_flop(self) -> float:
        # two contractions of length D per allowed pair (QK^T and PV), 2 flop per MAC
        return 4.0 * self.batch * self.heads_q * self.head_dim * self.allowed_pairs_per_head()

    def bwd_flop(self) -> float:
        # five contractions per allowed pair: QK^T recompute, dO V^T, P^T dO, dS^T Q, dS K
        return 10.0 * self.batch * self.heads_q * self.head_dim * self.allowed_pairs_per_head()


CONFIGS = {
    "ring_small_d64": Workload(
        "ring_small_d64", 1, 4, 4, 1024, 64, n_chunks=4,
        description="B1 H4 S1024 D64, 4 ring chunks of 256 in seeded random order"),
    "llama2_7b_s32k_ring8": Workload(
        "llama2_7b_s32k_ring8", 1, 32, 32, 32768, 128, n_chunks=8,
        description="Llama-2-7B attention shape, S=32768, 8 ring chunks of 4096, forward"),
    "s2attn_llama2_7b_s8k_g2048": Workload(
        "s2attn_llama2_7b_s8k_g2048", 1, 32, 32, 8192, 128, s2_group=2048, s2_shift_head0=16,
        backward=True,
        description="S2-Attn at Llama-2-7B shape, S=8192, group 2048, heads 16-31 shifted by 1024"),
    "gqa_llama3_8b_s128k_ring16": Workload(
        "gqa_llama3_8b_s128k_ring16", 1, 32, 8, 131072, 128, n_chunks=16,
        description="Llama-3-8B GQA (32 q heads, 8 kv heads), S=131072, 16 ring chunks of 8192, forward"),
    "s2attn_llama2_7b_s100k_g25600": Workload(
        "s2attn_llama2_7b_s100k_g25600", 1, 32, 32, 102400, 128, s2_group=25600, s2_shift_head0=16,
        backward=True,
        description="S2-Attn at long context: Llama-2-7B shape, S=102400, group S/4=25600, heads 16-31 "
                    "shifted by 12800, forward + backward"),
    "llama2_13b_s64k_ring8_train": Workload(
        "llama2_13b_s64k_ring8_train", 1, 40, 40, 65536, 128, n_chunks=8, backward=True,
        description="Llama-2-13B attention shape, S=65536, 8 ring chunks of 8192, forward + backward"),
}

# short aliases in the order the workloads are listed above
ALIASES = {
    "c1": "ring_small_d64",
    "c2": "llama2_7b_s32k_ring8",
    "c3": "s2attn_llama2_7b_s8k_g2048",
    "c4": "gqa_llama3_8b_s128k_ring16",
    "c5": "llama2_13b_s64k_ring8_train",
    "s2_100k": "s2attn_llama2_7b_s100k_g25600",
}


def get(name: str) -> Workload:
    name = ALIASES.get(name, name)
    return CONFIGS[name]


@dataclass(frozen=True)
class FfnWorkload:
    """Blockwise feedforward (SwiGLU) of `rows` query rows, `block_rows` at a time."""
    name: str
    rows: int
    d_model: int
    d_ff: int
    block_rows: int
    seed: int = 0
    description: str = ""

    def flop(self) -> float:
        # three GEMMs of rows x d_model x d_ff, 2 flop per MAC
        return 6.0 * self.rows * self.d_model * self.d_ff


FFN_CONFIGS = {
    "ffn_llama2_7b_s32k": FfnWorkload(
        "ffn_llama2_7b_s32k", 32768, 4096, 11008, 4096,
        description="Llama-2-7B SwiGLU feedforward (d_model 4096, d_ff 11008) of the 32768 rows of the "
                    "32K attention workload, in blocks of 4096 rows"),
}
