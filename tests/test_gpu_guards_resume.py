"""CPU-side checks of what the GPU path writes, and of the ring state as a resumable checkpoint.

Guard bands: every output of a ring forward and backward is carved from the middle of a larger
buffer whose margins hold a canary bit pattern; after the calls the margins must be unchanged,
so no kernel writes past either end of an output (a ragged shape puts partial tiles at the end).

Resume: on a ring, the running pair (O_acc, LSE) after k steps is the whole state of the forward
(the Ring Attention summary, Summary: blocks combine in any order, one at a time), and dQ_acc (with
delta) the whole state of the backward.  Stopping after k steps, copying the state to the host,
reloading it into fresh device memory and finishing must give the uninterrupted result bit for bit.
"""
import numpy as np
import pytest
import torch

import long_context_exact_blockattn_amd as ba
from long_context_exact_blockattn_amd import _lib
from oracle import attention_forward
from tests.gpu_helpers import TOL_LSE, TOL_O, dev, f64, log, max_err
from workloads import chunk_bounds, chunk_order, make_inputs

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements of margin on each side
CANARY32 = 0x7FC0DEAD  # a NaN payload no kernel produces
CANARY16 = 0x7FA5


def _guarded(shape, dtype):
    """(view of `shape` in the middle of a larger buffer, the whole buffer)."""
    n = int(np.prod(shape))
    if dtype == torch.float32:
        buf = torch.full((n + 2 * GUARD,), CANARY32, dtype=torch.int32, device=dev())
    else:
        buf = torch.full((n + 2 * GUARD,), CANARY16, dtype=torch.int16, device=dev())
    return buf[GUARD:GUARD + n].view(dtype).view(shape), buf


def _margins_intact(buf, name):
    canary = CANARY32 if buf.dtype == torch.int32 else CANARY16
    lo, hi = buf[:GUARD].cpu(), buf[-GUARD:].cpu()
    bad = int((lo != canary).sum()) + int((hi != canary).sum())
    assert bad == 0, f"{bad} guard elements of {name} overwritten"


@pytest.mark.parametrize("D", [64, 128])
def test_guard_bands_around_every_output(D):
    B, S, Hq, Hkv, n = 2, 333, 4, 2, 3
    q, k, v, do = make_inputs(B, S, Hq, Hkv, D, seed=400 + D, with_dout=True)
    qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
    o_acc, g_oacc = _guarded((B, S, Hq, D), torch.float32)
    lse, g_lse = _guarded((B, Hq, S), torch.float32)
    out, g_out = _guarded((B, S, Hq, D), torch.bfloat16)
    delta, g_delta = _guarded((B, Hq, S), torch.float32)
    dq_acc, g_dqacc = _guarded((B, S, Hq, D), torch.float32)
    dq, g_dq = _guarded((B, S, Hq, D), torch.bfloat16)
    dk, g_dk = _guarded((B, S, Hkv, D), torch.bfloat16)
    dv, g_dv = _guarded((B, S, Hkv, D), torch.bfloat16)
    dq_acc.zero_()
    order = chunk_order(n, seed=2)
    bounds = chunk_bounds(S, n)
    for t, c in enumerate(order):
        c0, c1 = bounds[c]
        _lib.blockattn_fwd(qd, kd[:, c0:c1], vd[:, c0:c1], o_acc, lse,
                           mode=_lib.BA_OVERWRITE if t == 0 else _lib.BA_ACCUMULATE,
                           o_final=out if t == n - 1 else None, k_pos0=c0)
    for t, c in enumerate(order):
        c0, c1 = bounds[c]
        flags = (_lib.BA_BWD_COMPUTE_DELTA if t == 0 else 0) | (_lib.BA_BWD_FINALIZE_DQ if t == n - 1 else 0)
        _lib.blockattn_bwd(qd, kd[:, c0:c1], vd[:, c0:c1], out, dod, lse, delta, dq_acc, dk[:, c0:c1],
                           dv[:, c0:c1], dq_final=dq, flags=flags, k_pos0=c0)
    torch.cuda.synchronize()
    for buf, name in ((g_oacc, "o_acc"), (g_lse, "lse"), (g_out, "out"), (g_delta, "delta"),
                      (g_dqacc, "dq_acc"), (g_dq, "dq"), (g_dk, "dk"), (g_dv, "dv")):
        _margins_intact(buf, name)
    # and the outputs themselves were written and are right
    o_ref, l_ref = attention_forward(f64(q), f64(k), f64(v))
    eo, el = max_err(o_acc, o_ref), max_err(lse, l_ref)
    log(f"guarded outputs D={D}: margins intact; max|O-ref| {eo:.3e} max|LSE-ref| {el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE
    for t in (dq, dk, dv):
        assert not torch.isnan(t).any()


@pytest.mark.parametrize("stop_after", [1, 3])
def test_ring_resumed_from_host_copy_is_bit_identical(stop_after):
    B, S, Hq, Hkv, D, n = 1, 1024, 4, 2, 128, 4
    q, k, v, do = make_inputs(B, S, Hq, Hkv, D, seed=500, with_dout=True)
    qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
    order = chunk_order(n, seed=7)
    bounds = chunk_bounds(S, n)

    def fwd_steps(o_acc, lse, out, steps):
        for t in steps:
            c0, c1 = bounds[order[t]]
            _lib.blockattn_fwd(qd, kd[:, c0:c1], vd[:, c0:c1], o_acc, lse,
                               mode=_lib.BA_OVERWRITE if t == 0 else _lib.BA_ACCUMULATE,
                               o_final=out if t == n - 1 else None, k_pos0=c0)

    def bwd_steps(out, lse, delta, dq_acc, dq, dk, dv, steps):
        for t in steps:
            c0, c1 = bounds[order[t]]
            flags = (_lib.BA_BWD_COMPUTE_DELTA if t == 0 else 0) | (_lib.BA_BWD_FINALIZE_DQ if t == n - 1 else 0)
            _lib.blockattn_bwd(qd, kd[:, c0:c1], vd[:, c0:c1], out, dod, lse, delta, dq_acc, dk[:, c0:c1],
                               dv[:, c0:c1], dq_final=dq, flags=flags, k_pos0=c0)

    new = lambda shape, dt=torch.float32: torch.empty(shape, device=dev(), dtype=dt)
    # uninterrupted
    o_acc, lse, out = new((B, S, Hq, D)), new((B, Hq, S)), new((B, S, Hq, D), torch.bfloat16)
    fwd_steps(o_acc, lse, out, range(n))
    delta, dq_acc = new((B, Hq, S)), torch.zeros(B, S, Hq, D, device=dev())
    dq, dk, dv = new((B, S, Hq, D), torch.bfloat16), new((B, S, Hkv, D), torch.bfloat16), new((B, S, Hkv, D), torch.bfloat16)
    bwd_steps(out, lse, delta, dq_acc, dq, dk, dv, range(n))
    torch.cuda.synchronize()

    # forward stopped after `stop_after` steps, state to the host, device copies dropped
    o2, l2, out2 = new((B, S, Hq, D)), new((B, Hq, S)), new((B, S, Hq, D), torch.bfloat16)
    fwd_steps(o2, l2, out2, range(stop_after))
    torch.cuda.synchronize()
    host = (o2.cpu(), l2.cpu())
    del o2, l2
    o3, l3 = host[0].to(dev()), host[1].to(dev())
    fwd_steps(o3, l3, out2, range(stop_after, n))
    torch.cuda.synchronize()
    assert torch.equal(o3, o_acc) and torch.equal(l3, lse) and torch.equal(out2, out)

    # backward stopped likewise: dq_acc and delta are its state (dk, dv of finished chunks are outputs)
    d2, a2 = new((B, Hq, S)), torch.zeros(B, S, Hq, D, device=dev())
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    bwd_steps(out, lse, d2, a2, dq2, dk2, dv2, range(stop_after))
    torch.cuda.synchronize()
    host = (d2.cpu(), a2.cpu())
    del d2, a2
    d3, a3 = host[0].to(dev()), host[1].to(dev())
    bwd_steps(out, lse, d3, a3, dq2, dk2, dv2, range(stop_after, n))
    torch.cuda.synchronize()
    assert torch.equal(a3, dq_acc) and torch.equal(dq2, dq)
    assert torch.equal(dk2, dk) and torch.equal(dv2, dv)
    log(f"ring resumed after {stop_after} of {n} steps from a host copy: forward and backward bit-identical")
