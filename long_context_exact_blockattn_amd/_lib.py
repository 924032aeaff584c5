"""ctypes binding of libblockattn.so: argument marshalling only.

Every function here takes torch tensors that already live on the GPU, checks
that their shapes and strides fit the C ABI (include/blockattn.h), passes raw
device pointers, element strides and the current HIP stream, and raises if the
library returns an error status.  All arithmetic runs in the library's HIP
kernels; there is no CPU fallback, and importing this module fails loudly when
the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libblockattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "blockattn.h")

BA_OK = 0
BA_ERR_NULL, BA_ERR_SHAPE, BA_ERR_STRIDE, BA_ERR_ALIGN = 1, 2, 3, 4
BA_ERR_UNSUPPORTED, BA_ERR_S2, BA_ERR_MODE, BA_ERR_LAUNCH = 5, 6, 7, 8
BA_ERR_WORKSPACE = 9
NOALLOC_MAX_ROWS = 1 << 23  # BLOCKATTN_NOALLOC_MAX_ROWS
BA_F32, BA_BF16 = 0, 1
BA_OVERWRITE, BA_ACCUMULATE = 0, 1
BA_FINAL_REACHED_ONLY = 4  # flag OR-ed into the forward mode
BA_BWD_COMPUTE_DELTA, BA_BWD_FINALIZE_DQ = 1, 2


class BaDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int64),
        ("seqlen_k", ctypes.c_int64),
        ("q_pos0", ctypes.c_int64),
        ("k_pos0", ctypes.c_int64),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q_stride", ctypes.c_int64 * 3),
        ("kv_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
    ]


class BaS2Desc(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("shift_head0", ctypes.c_int32)]


class BlockAttnError(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


_lib = None


def load():
    """Load libblockattn.so (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first (python -c "
            "'import __graft_entry__; __graft_entry__.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(BaDesc)
    S2 = ctypes.POINTER(BaS2Desc)
    i32 = ctypes.c_int32
    lib.blockattn_fwd.argtypes = [D, P, P, P, P, i32, P, i32, P, P]
    lib.blockattn_fwd.restype = ctypes.c_int
    lib.lse_merge.argtypes = [D, P, P, P, i32, P, P, P]
    lib.lse_merge.restype = ctypes.c_int
    lib.blockattn_bwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, i32, P, i32, P]
    lib.blockattn_bwd.restype = ctypes.c_int
    lib.blockattn_bwd_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, i32, P, i32, P]
    lib.blockattn_bwd_noalloc.restype = ctypes.c_int
    lib.s2attn_fwd.argtypes = [D, S2, P, P, P, P, i32, P, P]
    lib.s2attn_fwd.restype = ctypes.c_int
    lib.s2attn_bwd.argtypes = [D, S2, P, P, P, P, P, P, P, P, P, P, i32, P, i32, P]
    lib.s2attn_bwd.restype = ctypes.c_int
    i64 = ctypes.c_int64
    for fn in (lib.ulysses_pack, lib.ulysses_unpack):
        fn.argtypes = [P, P, i64, i64, i32, i32, i32, P]
        fn.restype = ctypes.c_int
    lib.bpt_ffn.argtypes = [P, P, P, P, P, P, i64, i32, i32, i64, P]
    lib.bpt_ffn.restype = ctypes.c_int
    lib.blockattn_status_string.argtypes = [ctypes.c_int]
    lib.blockattn_status_string.restype = ctypes.c_char_p
    lib.blockattn_debug_fwd_schedule.argtypes = [D, S2, i32, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64]
    lib.blockattn_debug_fwd_schedule.restype = ctypes.c_int64
    lib.blockattn_debug_tile_sizes.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.blockattn_debug_tile_sizes.restype = ctypes.c_int
    _lib = lib
    return lib


def header_functions():
    """Names of the functions include/blockattn.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)) - {"if"})


def status_string(status):
    return load().blockattn_status_string(int(status)).decode()


def _check(status, fn):
    if status != BA_OK:
        raise BlockAttnError(status, fn)


# ---------------------------------------------------------------- marshalling helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(ref, specs):
    """Every tensor of specs [(tensor or None, name, dtype name or None)] must live on ref's GPU
    and have the named dtype: the kernels take raw device pointers and size every access from
    the descriptor, so a host tensor or a narrower dtype would be read or written out of bounds."""
    import torch
    if not ref.is_cuda:
        raise ValueError("tensors must be on a GPU (got a host tensor)")
    for t, name, dt in specs:
        if t is None:
            continue
        if not t.is_cuda or t.device != ref.device:
            raise ValueError(f"{name} must be on {ref.device} (got {t.device})")
        if dt is not None and t.dtype != getattr(torch, dt):
            raise ValueError(f"{name} must be {dt} (got {t.dtype})")


def _stream(stream):
    """A hipStream_t from None (torch's current stream), a torch stream, or a raw handle."""
    if stream is not None:
        return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _bshd_strides(t, name):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, S, H, D]")
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have a contiguous last (D) axis")
    return (t.stride(0), t.stride(1), t.stride(2))


def _same_layout(ref, t, name, shape=None, ref_name="o"):
    """t has ref's shape and, on every axis longer than one, ref's stride: the kernels address the
    tensors of one stride group (q; k, v, dk, dv; o, o_final, dout, dq_acc, dq_final) with one set
    of strides, and an axis of length one is never stepped along (torch keeps arbitrary strides
    there, e.g. after .contiguous() of a slice of a batch of one)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(ref.shape if shape is None else shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")
    if t.dim() == 4:
        ts, rs = _bshd_strides(t, name), _bshd_strides(ref, ref_name)
        if any(n > 1 and a != b for n, a, b in zip(t.shape[:3], ts, rs)):
            raise ValueError(f"{name} must have the same (b, s, h) strides as {ref_name}")


def _stats_ok(t, shape, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp32 tensor of shape {tuple(shape)}")


def make_desc(q, k, o=None, *, q_pos0=0, k_pos0=0, causal=True, scale=None):
    """Descriptor of a call: shapes from q and k, strides from q (q_stride), k (kv_stride) and
    o (o_stride: every other query-shaped tensor; q's own strides when o is None)."""
    if q.dim() != 4 or (k is not None and k.dim() != 4):
        raise ValueError("q and k must be [B, S, H, D]")
    b, sq, hq, d = q.shape
    if o is not None and tuple(o.shape) != tuple(q.shape):
        raise ValueError(f"o has shape {tuple(o.shape)}, expected {tuple(q.shape)}")
    # the descriptor carries one batch size and one head size for every tensor of the call
    if k is not None and (k.shape[0] != b or k.shape[3] != d):
        raise ValueError(f"k {tuple(k.shape)} must have q's batch ({b}) and head_dim ({d})")
    sk, hkv = (k.shape[1], k.shape[2]) if k is not None else (0, hq)
    desc = BaDesc()
    desc.batch, desc.heads_q, desc.heads_kv, desc.head_dim = b, hq, hkv, d
    desc.seqlen_q, desc.seqlen_k = sq, sk
    desc.q_pos0, desc.k_pos0 = int(q_pos0), int(k_pos0)
    desc.causal = 1 if causal else 0
    desc.scale = 0.0 if scale is None else float(scale)
    desc.q_stride[:] = _used_strides(q, "q")
    desc.kv_stride[:] = _used_strides(k, "k") if k is not None else (0, 0, 0)
    desc.o_stride[:] = _used_strides(q if o is None else o, "o")
    return desc


def _used_strides(t, name):
    """(b, s, h) strides with 0 on axes of length one: the kernels never step along those, and
    torch may leave any value there (which the library would check against its stride rules)."""
    return tuple(0 if n == 1 else st for n, st in zip(t.shape[:3], _bshd_strides(t, name)))


def _dtype_code(t, name):
    import torch
    if t.dtype == torch.float32:
        return BA_F32
    if t.dtype == torch.bfloat16:
        return BA_BF16
    raise ValueError(f"{name} must be float32 or bfloat16")


# ---------------------------------------------------------------- entry points

def blockattn_fwd(q, k, v, o, lse, *, mode=BA_OVERWRITE, o_final=None, q_pos0=0, k_pos0=0,
                  causal=True, scale=None, stream=None):
    """One ring step; see blockattn_fwd in include/blockattn.h."""
    _require(q, [(q, "q", "bfloat16"), (k, "k", "bfloat16"), (v, "v", "bfloat16"), (o, "o", None),
                 (lse, "lse", "float32"), (o_final, "o_final", "bfloat16")])
    desc = make_desc(q, k, o, q_pos0=q_pos0, k_pos0=k_pos0, causal=causal, scale=scale)
    _same_layout(k, v, "v", ref_name="k")
    _same_layout(o, o_final, "o_final")
    _stats_ok(lse, (q.shape[0], q.shape[2], q.shape[1]), "lse")
    st = load().blockattn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                              _dtype_code(o, "o"), _ptr(lse), int(mode), _ptr(o_final), _stream(stream))
    _check(st, "blockattn_fwd")


def lse_merge(o_acc, lse_acc, o_part, lse_part, *, o_final=None, stream=None):
    """(o_acc, lse_acc) := merge with (o_part, lse_part); see lse_merge in include/blockattn.h."""
    _require(o_acc, [(o_acc, "o_acc", "float32"), (lse_acc, "lse_acc", "float32"), (o_part, "o_part", None),
                     (lse_part, "lse_part", "float32"), (o_final, "o_final", "bfloat16")])
    desc = make_desc(o_acc, None, o_acc)
    _same_layout(o_acc, o_part, "o_part", ref_name="o_acc")
    _same_layout(o_acc, o_final, "o_final", ref_name="o_acc")
    shape = (o_acc.shape[0], o_acc.shape[2], o_acc.shape[1])
    _stats_ok(lse_acc, shape, "lse_acc")
    _stats_ok(lse_part, shape, "lse_part")
    st = load().lse_merge(ctypes.byref(desc), _ptr(o_acc), _ptr(lse_acc), _ptr(o_part),
                          _dtype_code(o_part, "o_part"), _ptr(lse_part), _ptr(o_final), _stream(stream))
    _check(st, "lse_merge")


def s2attn_fwd(q, k, v, o, lse, *, group, shift_head0, scale=None, stream=None):
    _require(q, [(q, "q", "bfloat16"), (k, "k", "bfloat16"), (v, "v", "bfloat16"), (o, "o", None),
                 (lse, "lse", "float32")])
    desc = make_desc(q, k, o, causal=True, scale=scale)
    _same_layout(k, v, "v", ref_name="k")
    _stats_ok(lse, (q.shape[0], q.shape[2], q.shape[1]), "lse")
    s2 = BaS2Desc(int(group), int(shift_head0))
    st = load().s2attn_fwd(ctypes.byref(desc), ctypes.byref(s2), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                           _dtype_code(o, "o"), _ptr(lse), _stream(stream))
    _check(st, "s2attn_fwd")


def _check_bwd(q, k, v, o, dout, lse, delta, dq_acc, dk, dv, dq_final):
    _require(q, [(q, "q", "bfloat16"), (k, "k", "bfloat16"), (v, "v", "bfloat16"), (o, "o", "bfloat16"),
                 (dout, "dout", "bfloat16"), (lse, "lse", "float32"), (delta, "delta", "float32"),
                 (dq_acc, "dq_acc", "float32"), (dk, "dk", None), (dv, "dv", None),
                 (dq_final, "dq_final", "bfloat16")])
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError(f"o has shape {tuple(o.shape)}, expected {tuple(q.shape)}")
    for t, n in ((dout, "dout"), (dq_acc, "dq_acc"), (dq_final, "dq_final")):
        _same_layout(o, t, n)
    for t, n in ((v, "v"), (dk, "dk"), (dv, "dv")):
        _same_layout(k, t, n, ref_name="k")
    if dk.dtype != dv.dtype:
        raise ValueError("dk and dv must share a dtype")
    shape = (q.shape[0], q.shape[2], q.shape[1])
    _stats_ok(lse, shape, "lse")
    _stats_ok(delta, shape, "delta")


def blockattn_bwd(q, k, v, o, dout, lse, delta, dq_acc, dk, dv, *, dq_final=None, flags=0,
                  q_pos0=0, k_pos0=0, causal=True, scale=None, stream=None):
    """One ring step of the backward; see blockattn_bwd in include/blockattn.h."""
    _check_bwd(q, k, v, o, dout, lse, delta, dq_acc, dk, dv, dq_final)
    desc = make_desc(q, k, o, q_pos0=q_pos0, k_pos0=k_pos0, causal=causal, scale=scale)
    st = load().blockattn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                              _ptr(lse), _ptr(delta), _ptr(dq_acc), _ptr(dk), _ptr(dv),
                              _dtype_code(dk, "dk"), _ptr(dq_final), int(flags), _stream(stream))
    _check(st, "blockattn_bwd")


def blockattn_bwd_noalloc(q, k, v, o, dout, lse, dq_acc, dk, dv, *, dq_final=None, flags=0, q_pos0=0,
                          k_pos0=0, causal=True, scale=None, stream=None):
    """blockattn_bwd with its delta rows in the library's static device buffer (no workspace
    argument, no allocation); delta is computed on every call.  See include/blockattn.h."""
    _check_bwd(q, k, v, o, dout, lse, None, dq_acc, dk, dv, dq_final)
    desc = make_desc(q, k, o, q_pos0=q_pos0, k_pos0=k_pos0, causal=causal, scale=scale)
    st = load().blockattn_bwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                      _ptr(lse), _ptr(dq_acc), _ptr(dk), _ptr(dv), _dtype_code(dk, "dk"),
                                      _ptr(dq_final), int(flags), _stream(stream))
    _check(st, "blockattn_bwd_noalloc")


def s2attn_bwd(q, k, v, o, dout, lse, delta, dq_acc, dk, dv, *, group, shift_head0, dq_final=None,
               flags=0, scale=None, stream=None):
    _check_bwd(q, k, v, o, dout, lse, delta, dq_acc, dk, dv, dq_final)
    desc = make_desc(q, k, o, causal=True, scale=scale)
    s2 = BaS2Desc(int(group), int(shift_head0))
    st = load().s2attn_bwd(ctypes.byref(desc), ctypes.byref(s2), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                           _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq_acc), _ptr(dk), _ptr(dv),
                           _dtype_code(dk, "dk"), _ptr(dq_final), int(flags), _stream(stream))
    _check(st, "s2attn_bwd")


def _dense_bf16(t, name, fn):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{fn}: {name} must be on a GPU (got a host tensor)")
    if t.dtype != torch.bfloat16:
        raise BlockAttnError(BA_ERR_UNSUPPORTED, f"{fn} ({name} must be bf16)")
    if not t.is_contiguous():
        raise BlockAttnError(BA_ERR_STRIDE, f"{fn} ({name} must be dense)")


def ulysses_pack(x, n_devices, *, send=None, stream=None):
    """x [B, Sl, H, D] -> send [N, B, Sl, H/N, D]; see ulysses_pack in include/blockattn.h."""
    import torch
    _dense_bf16(x, "x", "ulysses_pack")
    b, sl, h, d = x.shape
    if n_devices < 1 or h % n_devices != 0:
        raise BlockAttnError(BA_ERR_SHAPE, "ulysses_pack (heads must split evenly over n_devices)")
    if send is None:
        send = torch.empty((n_devices, b, sl, h // n_devices, d), device=x.device, dtype=x.dtype)
    _dense_bf16(send, "send", "ulysses_pack")
    if send.numel() != x.numel():
        raise BlockAttnError(BA_ERR_SHAPE, "ulysses_pack (send must hold as many elements as x)")
    st = load().ulysses_pack(_ptr(x), _ptr(send), b, sl, h, d, n_devices, _stream(stream))
    _check(st, "ulysses_pack")
    return send


def ulysses_unpack(recv, n_devices, *, x=None, stream=None):
    """recv [N, B, Sl, H/N, D] -> x [B, Sl, H, D]; see ulysses_unpack in include/blockattn.h."""
    import torch
    _dense_bf16(recv, "recv", "ulysses_unpack")
    n, b, sl, hn, d = recv.shape
    if n != n_devices:
        raise BlockAttnError(BA_ERR_SHAPE, "ulysses_unpack (recv's first axis must be n_devices)")
    if x is None:
        x = torch.empty((b, sl, hn * n, d), device=recv.device, dtype=recv.dtype)
    _dense_bf16(x, "x", "ulysses_unpack")
    if x.numel() != recv.numel():
        raise BlockAttnError(BA_ERR_SHAPE, "ulysses_unpack (x must hold as many elements as recv)")
    st = load().ulysses_unpack(_ptr(recv), _ptr(x), b, sl, hn * n, d, n_devices, _stream(stream))
    _check(st, "ulysses_unpack")
    return x


def bpt_ffn(x, w1, w3, w2, *, block_rows=4096, out=None, hidden=None, stream=None):
    """SwiGLU feedforward of the rows of x [rows, d_model], block by block; see bpt_ffn in
    include/blockattn.h.  hidden is the [block_rows, d_ff] workspace (allocated if None)."""
    import torch
    for name, t in (("x", x), ("w1", w1), ("w3", w3), ("w2", w2)):
        _dense_bf16(t, name, "bpt_ffn")
    rows, d_model = x.shape
    d_ff = w1.shape[0]
    if w1.shape != (d_ff, d_model) or w3.shape != (d_ff, d_model) or w2.shape != (d_model, d_ff):
        raise BlockAttnError(BA_ERR_SHAPE, "bpt_ffn (w1, w3 must be [d_ff, d_model], w2 [d_model, d_ff])")
    if out is None:
        out = torch.empty_like(x)
    if hidden is None:
        hidden = torch.empty((min(block_rows, max(rows, 1)), d_ff), device=x.device, dtype=x.dtype)
    _dense_bf16(out, "out", "bpt_ffn")
    _dense_bf16(hidden, "hidden", "bpt_ffn")
    if out.shape != x.shape or hidden.numel() < min(block_rows, rows) * d_ff:
        raise BlockAttnError(BA_ERR_SHAPE, "bpt_ffn (out must match x; hidden must hold block_rows x d_ff)")
    st = load().bpt_ffn(_ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out), _ptr(hidden), rows, d_model, d_ff,
                        block_rows, _stream(stream))
    _check(st, "bpt_ffn")
    return out


def debug_fwd_schedule(desc, head, s2=None):
    """Host-side enumeration of the forward tile schedule: int64 array [n, 4]."""
    import numpy as np
    lib = load()
    s2p = ctypes.byref(s2) if s2 is not None else None
    n = lib.blockattn_debug_fwd_schedule(ctypes.byref(desc), s2p, int(head), None, 0)
    if n < 0:
        raise BlockAttnError(-n, "blockattn_debug_fwd_schedule")
    buf = (ctypes.c_int64 * (4 * max(n, 1)))()
    lib.blockattn_debug_fwd_schedule(ctypes.byref(desc), s2p, int(head), buf, n)
    return np.frombuffer(buf, dtype=np.int64, count=4 * n).reshape(n, 4).copy()


def debug_tile_sizes(head_dim):
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    _check(load().blockattn_debug_tile_sizes(int(head_dim), ctypes.byref(bq), ctypes.byref(bk)),
           "blockattn_debug_tile_sizes")
    return bq.value, bk.value
