"""The allocation-free backward entry point (blockattn_bwd_noalloc) against blockattn_bwd.

The variant keeps delta in the library's static device buffer and computes it on every call; it
runs the same kernels, so every output must equal blockattn_bwd's bit for bit.  Two problems in a
row, the second smaller, show that the buffer's leftover contents from the first do not leak into
the second; a ring of chunks shows the per-call use.
"""
import pytest
import torch

from long_context_exact_blockattn_amd import _lib
from tests.gpu_helpers import dev, log
from workloads import chunk_bounds, chunk_order, make_inputs

pytestmark = pytest.mark.gpu


def _both(q, k, v, o, do, lse, flags, **kw):
    """(dq_acc, dq, dk, dv) from blockattn_bwd and from blockattn_bwd_noalloc on the same inputs."""
    res = []
    for noalloc in (False, True):
        B, S, Hq, D = q.shape
        dq_acc = torch.zeros(B, S, Hq, D, device=dev())
        dq = torch.full((B, S, Hq, D), float("nan"), device=dev(), dtype=torch.bfloat16)
        dk = torch.full(k.shape, float("nan"), device=dev(), dtype=torch.bfloat16)
        dv = torch.full(v.shape, float("nan"), device=dev(), dtype=torch.bfloat16)
        if noalloc:
            _lib.blockattn_bwd_noalloc(q, k, v, o, do, lse, dq_acc, dk, dv, dq_final=dq, flags=flags, **kw)
        else:
            delta = torch.empty(B, Hq, S, device=dev())
            _lib.blockattn_bwd(q, k, v, o, do, lse, delta, dq_acc, dk, dv, dq_final=dq,
                               flags=flags | _lib.BA_BWD_COMPUTE_DELTA, **kw)
        torch.cuda.synchronize()
        res.append((dq_acc, dq, dk, dv))
    return res


def _fwd(q, k, v):
    B, S, Hq, D = q.shape
    o_acc = torch.empty(B, S, Hq, D, device=dev())
    lse = torch.empty(B, Hq, S, device=dev())
    o = torch.empty(B, S, Hq, D, device=dev(), dtype=torch.bfloat16)
    _lib.blockattn_fwd(q, k, v, o_acc, lse, o_final=o)
    return o, lse


def test_noalloc_equals_backward_on_two_calls_second_smaller():
    for tag, (B, S, Hq, Hkv, D) in (("first", (2, 1500, 8, 2, 128)), ("second, smaller", (1, 333, 4, 4, 64))):
        q, k, v, do = (t.to(dev()) for t in make_inputs(B, S, Hq, Hkv, D, seed=S, with_dout=True))
        o, lse = _fwd(q, k, v)
        ref, got = _both(q, k, v, o, do, lse, _lib.BA_BWD_FINALIZE_DQ)
        for name, a, b in zip(("dq_acc", "dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), f"{tag} call: {name} differs from blockattn_bwd"
        log(f"noalloc {tag} call (B{B} S{S} Hq{Hq} Hkv{Hkv} D{D}): bit-identical to blockattn_bwd")


def test_noalloc_ring_equals_backward_ring():
    B, S, Hq, Hkv, D, n = 1, 1024, 4, 2, 128, 3
    q, k, v, do = (t.to(dev()) for t in make_inputs(B, S, Hq, Hkv, D, seed=9, with_dout=True))
    o, lse = _fwd(q, k, v)
    order = chunk_order(n, seed=4)
    bounds = chunk_bounds(S, n)
    outs = []
    for noalloc in (False, True):
        dq_acc = torch.zeros(B, S, Hq, D, device=dev())
        dq = torch.empty(B, S, Hq, D, device=dev(), dtype=torch.bfloat16)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        delta = torch.empty(B, Hq, S, device=dev())
        for t, c in enumerate(order):
            c0, c1 = bounds[c]
            flags = (_lib.BA_BWD_COMPUTE_DELTA if t == 0 else 0) | (_lib.BA_BWD_FINALIZE_DQ if t == n - 1 else 0)
            if noalloc:
                _lib.blockattn_bwd_noalloc(q, k[:, c0:c1], v[:, c0:c1], o, do, lse, dq_acc, dk[:, c0:c1],
                                           dv[:, c0:c1], dq_final=dq, flags=flags, k_pos0=c0)
            else:
                _lib.blockattn_bwd(q, k[:, c0:c1], v[:, c0:c1], o, do, lse, delta, dq_acc, dk[:, c0:c1],
                                   dv[:, c0:c1], dq_final=dq, flags=flags, k_pos0=c0)
        torch.cuda.synchronize()
        outs.append((dq_acc, dq, dk, dv))
    for name, a, b in zip(("dq_acc", "dq", "dk", "dv"), *outs):
        assert torch.equal(a, b), f"ring: {name} differs"
    log(f"noalloc ring of {n} chunks: bit-identical to blockattn_bwd")
