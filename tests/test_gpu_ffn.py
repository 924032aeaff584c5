"""GPU parity of the blockwise feedforward (bpt_ffn) against the oracle's SwiGLU definition.

Gate: relative L2 error <= 1e-2 per output (the kernel rounds the hidden activation and the output
to bf16, ~2^-9 relative each, against an fp64 oracle on the same bf16 inputs), plus the maximum
absolute error <= 2^-6 times the output's maximum magnitude.
"""
import numpy as np
import pytest
import torch

import long_context_exact_blockattn_amd as ba
from oracle.ffn import swiglu_ffn
from tests.gpu_helpers import dev, log, rel_l2
from workloads import FFN_CONFIGS, make_ffn_inputs

pytestmark = pytest.mark.gpu

TOL_FFN = 1e-2


def _check(tag, got, ref):
    got = got.float().cpu().numpy().astype(np.float64)
    err = rel_l2(torch.from_numpy(got), ref)
    amax = float(np.abs(got - ref).max())
    log(f"{tag}: rel L2 {err:.3e}, max abs {amax:.3e} (output max {np.abs(ref).max():.3f})")
    assert err <= TOL_FFN and amax <= np.abs(ref).max() / 64


# (1300, ..., 1300): six row tiles, so the item order's groups of four row tiles end in a
# partial group of two
@pytest.mark.parametrize("rows,d_model,d_ff,block_rows", [(1000, 256, 384, 300), (256, 512, 128, 256),
                                                          (77, 256, 256, 1000), (1300, 256, 384, 1300)])
def test_ffn_small(rows, d_model, d_ff, block_rows):
    x, w1, w3, w2 = make_ffn_inputs(rows, d_model, d_ff, seed=rows)
    out = ba.bpt_ffn(*(t.to(dev()) for t in (x, w1, w3, w2)), block_rows=block_rows)
    torch.cuda.synchronize()
    _check(f"ffn rows={rows} d={d_model} f={d_ff} block={block_rows}", out,
           swiglu_ffn(x.float().numpy(), w1.float().numpy(), w3.float().numpy(), w2.float().numpy()))


def test_ffn_blocking_does_not_change_bits():
    x, w1, w3, w2 = (t.to(dev()) for t in make_ffn_inputs(1200, 256, 384, seed=3))
    a = ba.bpt_ffn(x, w1, w3, w2, block_rows=1200)
    b = ba.bpt_ffn(x, w1, w3, w2, block_rows=256)
    c = ba.bpt_ffn(x, w1, w3, w2, block_rows=333)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_ffn_llama2_7b_shape_sampled_rows():
    w = FFN_CONFIGS["ffn_llama2_7b_s32k"]
    x, w1, w3, w2 = make_ffn_inputs(w.rows, w.d_model, w.d_ff, seed=w.seed)
    out = ba.bpt_ffn(*(t.to(dev()) for t in (x, w1, w3, w2)), block_rows=w.block_rows)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 4095, 4096, w.rows - 1, *map(int, np.random.default_rng(4).integers(0, w.rows, 11))})
    ref = swiglu_ffn(x[rows].float().numpy(), w1.float().numpy(), w3.float().numpy(), w2.float().numpy())
    _check(f"ffn Llama-2-7B shape, {len(rows)} sampled rows of {w.rows}", out[rows], ref)
