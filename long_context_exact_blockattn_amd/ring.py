"""Ring steps on one GPU: the resident query block against key/value chunks in a given order.

On a ring of hosts (Ring Attention summary, Summary) each host keeps its query
block while key/value blocks arrive one per step; here the chunks are visited
sequentially on one device, in any order, and every step is one library call
that merges its partial (O, LSE) pair into the running pair.
"""
from __future__ import annotations

import torch

from . import _lib


def _bounds(seqlen_k, n_chunks):
    c = -(-seqlen_k // n_chunks)
    return [(i * c, min((i + 1) * c, seqlen_k)) for i in range(n_chunks) if i * c < seqlen_k]


def final_store_steps(order, causal=True):
    """Which ring positions store the final bf16 output, and for which rows.

    Under the causal mask, chunk c reaches exactly the rows from its own start on, so a row's
    last reaching step is the last position whose chunk is at or before the row's block: the
    rows of blocks [c_t, min of the later chunks) are final after position t.  Those positions
    (each one whose chunk precedes every later chunk, always the last) pass o_final with
    BA_FINAL_REACHED_ONLY and store every row they reach, so each row's final output is stored
    by its last reaching step and no step converts the rows it cannot reach.  Without the mask
    every step reaches every row: only the last one stores.
    Returns one bool per position.
    """
    n = len(order)
    if not causal:
        return [t == n - 1 for t in range(n)]
    flags, later_min = [False] * n, n
    for t in range(n - 1, -1, -1):
        flags[t] = order[t] < later_min
        later_min = min(later_min, order[t])
    return flags


def _step_mode(t, store, causal):
    mode = _lib.BA_OVERWRITE if t == 0 else _lib.BA_ACCUMULATE
    return mode | _lib.BA_FINAL_REACHED_ONLY if (store and causal) else mode


def ring_forward(q, k, v, n_chunks, order=None, *, causal=True, scale=None, o_acc=None, lse=None,
                 out=None, stream=None):
    """Forward over `n_chunks` key/value chunks visited in `order`.

    Returns (out bf16 [B,S,Hq,D], lse fp32 [B,Hq,S], o_acc fp32 [B,S,Hq,D]).
    Step 0 overwrites the running pair (rows its chunk cannot reach become the
    empty pair (0, -inf)); later steps accumulate; the final bf16 output of each
    row is stored by its last reaching step (final_store_steps).
    """
    bounds = _bounds(k.shape[1], n_chunks)
    order = list(range(len(bounds))) if order is None else list(order)
    if sorted(order) != list(range(len(bounds))):
        raise ValueError("order must be a permutation of the chunk indices")
    b, s, hq, d = q.shape
    if o_acc is None:
        o_acc = torch.empty(b, s, hq, d, device=q.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty(b, hq, s, device=q.device, dtype=torch.float32)
    if out is None:
        out = torch.empty(b, s, hq, d, device=q.device, dtype=torch.bfloat16)
    store = final_store_steps(order, causal)
    for t, c in enumerate(order):
        c0, c1 = bounds[c]
        _lib.blockattn_fwd(q, k[:, c0:c1], v[:, c0:c1], o_acc, lse, mode=_step_mode(t, store[t], causal),
                           o_final=out if store[t] else None,
                           k_pos0=c0, causal=causal, scale=scale, stream=stream)
    return out, lse, o_acc


_COPY_STREAMS = {}  # device index -> the side stream staged rings copy on (created once)


def _copy_stream(device):
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    if idx not in _COPY_STREAMS:
        _COPY_STREAMS[idx] = torch.cuda.Stream(device=idx)  # default priority
    return _COPY_STREAMS[idx]


def ring_forward_staged(q, k, v, n_chunks, order=None, *, causal=True, scale=None, copy_stream=None):
    """ring_forward with every step's key/value chunk first copied into one of two staging buffers
    on a second stream, the copy for step t+1 running while step t computes.

    This is the receive side of a ring on one device: on a ring of hosts the next block arrives
    over the interconnect while the current one is being used (Ring Attention summary, Summary),
    and the method has no overhead when the compute of a step outlasts the transfer of a block.
    Here the transfer is a device-to-device copy of the same bytes.  The compute of step t waits
    for the copy of its chunk (event); the copy into a staging buffer waits for the compute that
    last read it (event), so the two buffers alternate.  Both streams have the default priority;
    without copy_stream the copies run on one side stream per device, created on first use.
    Returns (out bf16, lse fp32, o_acc fp32), equal bit for bit to ring_forward's.
    """
    bounds = _bounds(k.shape[1], n_chunks)
    order = list(range(len(bounds))) if order is None else list(order)
    if sorted(order) != list(range(len(bounds))):
        raise ValueError("order must be a permutation of the chunk indices")
    b, s, hq, d = q.shape
    main = torch.cuda.current_stream(q.device)
    side = _copy_stream(q.device) if copy_stream is None else copy_stream
    cmax = max(c1 - c0 for c0, c1 in bounds)
    kbuf = [torch.empty(b, cmax, k.shape[2], d, device=k.device, dtype=k.dtype) for _ in range(2)]
    vbuf = [torch.empty(b, cmax, v.shape[2], d, device=v.device, dtype=v.dtype) for _ in range(2)]
    o_acc = torch.empty(b, s, hq, d, device=q.device, dtype=torch.float32)
    lse = torch.empty(b, hq, s, device=q.device, dtype=torch.float32)
    out = torch.empty(b, s, hq, d, device=q.device, dtype=torch.bfloat16)
    copied = [torch.cuda.Event() for _ in range(2)]
    computed = [torch.cuda.Event() for _ in range(2)]
    side.wait_stream(main)  # the inputs and the buffers exist before any copy reads or fills them

    def copy(t):
        slot = t % 2
        c0, c1 = bounds[order[t]]
        with torch.cuda.stream(side):
            if t >= 2:
                side.wait_event(computed[slot])
            kbuf[slot][:, : c1 - c0].copy_(k[:, c0:c1], non_blocking=True)
            vbuf[slot][:, : c1 - c0].copy_(v[:, c0:c1], non_blocking=True)
            copied[slot].record(side)

    store = final_store_steps(order, causal)
    copy(0)
    for t in range(len(order)):
        slot = t % 2
        c0, c1 = bounds[order[t]]
        if t + 1 < len(order):
            copy(t + 1)
        main.wait_event(copied[slot])
        _lib.blockattn_fwd(q, kbuf[slot][:, : c1 - c0], vbuf[slot][:, : c1 - c0], o_acc, lse,
                           mode=_step_mode(t, store[t], causal), o_final=out if store[t] else None,
                           k_pos0=c0, causal=causal, scale=scale, stream=main)
        computed[slot].record(main)
    # the side stream read k and v and wrote the staging buffers: none of them may be
    # reused by the allocator before that stream's work is done
    for t in kbuf + vbuf + [k, v]:
        t.record_stream(side)
    return out, lse, o_acc


def _empty_in_layout(t, dtype):
    """An uninitialised tensor with t's shape and element strides (dense when t is): gradients of
    key-shaped tensors share k's strides in the C ABI.  A strided t (say a slice of a packed
    projection) gets storage spanning its strides, gaps included."""
    if t.is_contiguous():
        return torch.empty(t.shape, device=t.device, dtype=dtype)
    return torch.empty_strided(t.shape, t.stride(), device=t.device, dtype=dtype)


def ring_backward(q, k, v, o, dout, lse, n_chunks, order=None, *, causal=True, scale=None,
                  dkv_dtype=torch.bfloat16, dk=None, dv=None, stream=None):
    """Backward over key/value chunks: returns (dq bf16, dk, dv).

    The first step also computes delta = rowsum(dout * o); every step writes
    its chunk's dK, dV and adds into the fp32 dQ accumulator; the last step
    converts dQ to bf16.  dq and the fp32 accumulator take o's layout; dk and dv
    (allocated in k's layout unless given) must share k's strides.
    """
    bounds = _bounds(k.shape[1], n_chunks)
    order = list(range(len(bounds))) if order is None else list(order)
    if sorted(order) != list(range(len(bounds))):
        raise ValueError("order must be a permutation of the chunk indices")
    b, s, hq, d = q.shape
    delta = torch.empty(b, hq, s, device=q.device, dtype=torch.float32)
    dq_acc = _empty_in_layout(o, torch.float32).zero_()
    dq = _empty_in_layout(o, torch.bfloat16)
    dk = _empty_in_layout(k, dkv_dtype) if dk is None else dk
    dv = _empty_in_layout(k, dkv_dtype) if dv is None else dv
    for t, c in enumerate(order):
        c0, c1 = bounds[c]
        flags = 0
        if t == 0:
            flags |= _lib.BA_BWD_COMPUTE_DELTA
        if t == len(order) - 1:
            flags |= _lib.BA_BWD_FINALIZE_DQ
        _lib.blockattn_bwd(q, k[:, c0:c1], v[:, c0:c1], o, dout, lse, delta, dq_acc,
                           dk[:, c0:c1], dv[:, c0:c1], dq_final=dq, flags=flags, k_pos0=c0,
                           causal=causal, scale=scale, stream=stream)
    return dq, dk, dv
