"""Host-side tests of the C ABI: loading, exported symbols, validation, tile schedule.

No kernel runs here: every call either fails validation (so nothing is
enqueued) or is a host-only introspection entry point.
"""
import ctypes

import numpy as np
import pytest

from long_context_exact_blockattn_amd import _lib
from oracle import S2Spec, allowed_mask


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_library_exports_every_declared_symbol(lib):
    names = _lib.header_functions()
    assert {"blockattn_fwd", "blockattn_bwd", "lse_merge", "s2attn_fwd", "s2attn_bwd",
            "blockattn_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(0, 10):
        s = _lib.status_string(code)
        assert s.startswith("BA_"), s
    assert "unknown" in _lib.status_string(99)


def _desc(**kw):
    d = _lib.BaDesc()
    d.batch, d.heads_q, d.heads_kv, d.head_dim = kw.get("B", 1), kw.get("Hq", 2), kw.get("Hkv", 2), kw.get("D", 128)
    d.seqlen_q, d.seqlen_k = kw.get("Sq", 256), kw.get("Sk", 256)
    d.q_pos0, d.k_pos0 = kw.get("q0", 0), kw.get("k0", 0)
    d.causal, d.scale = kw.get("causal", 1), 0.0
    hq, hkv, D = d.heads_q, d.heads_kv, d.head_dim
    d.q_stride[:] = kw.get("qs", (d.seqlen_q * hq * D, hq * D, D))
    d.kv_stride[:] = kw.get("ks", (d.seqlen_k * hkv * D, hkv * D, D))
    d.o_stride[:] = kw.get("os", (d.seqlen_q * hq * D, hq * D, D))
    return d


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _fwd(lib, d, q=FAKE, k=FAKE, v=FAKE, o=FAKE, odt=_lib.BA_F32, lse=FAKE, mode=0, of=None):
    P = ctypes.c_void_p
    return lib.blockattn_fwd(ctypes.byref(d) if d is not None else None, P(q), P(k), P(v), P(o), odt,
                             P(lse), mode, P(of) if of else None, None)


def test_fwd_validation_codes(lib):
    assert _fwd(lib, None) == _lib.BA_ERR_NULL
    assert _fwd(lib, _desc(D=96)) == _lib.BA_ERR_UNSUPPORTED
    assert _fwd(lib, _desc(Hq=3, Hkv=2)) == _lib.BA_ERR_SHAPE
    assert _fwd(lib, _desc(Sq=-1)) == _lib.BA_ERR_SHAPE
    assert _fwd(lib, _desc(qs=(0, 12, 4))) == _lib.BA_ERR_STRIDE
    assert _fwd(lib, _desc(ks=(0, -8, 8))) == _lib.BA_ERR_STRIDE
    assert _fwd(lib, _desc(ks=(0, 1 << 24, 8))) == _lib.BA_ERR_STRIDE  # 32-bit tile offsets
    assert _fwd(lib, _desc(qs=(0, 1 << 24, 8))) == _lib.BA_ERR_STRIDE
    assert _fwd(lib, _desc(os=(0, 260, 8))) == _lib.BA_ERR_STRIDE
    assert _fwd(lib, _desc(os=(-8, 256, 8))) == _lib.BA_ERR_STRIDE
    assert _fwd(lib, _desc(os=(0, 1 << 24, 8))) == _lib.BA_ERR_STRIDE
    assert _fwd(lib, _desc(), q=FAKE + 2) == _lib.BA_ERR_ALIGN
    assert _fwd(lib, _desc(), lse=FAKE + 2) == _lib.BA_ERR_ALIGN
    assert _fwd(lib, _desc(), of=FAKE + 8) == _lib.BA_ERR_ALIGN
    assert _fwd(lib, _desc(), q=0) == _lib.BA_ERR_NULL
    assert _fwd(lib, _desc(), mode=2) == _lib.BA_ERR_MODE
    assert _fwd(lib, _desc(), mode=6) == _lib.BA_ERR_MODE  # a mode flag does not make 2 a mode
    assert _fwd(lib, _desc(), odt=_lib.BA_BF16, mode=_lib.BA_ACCUMULATE) == _lib.BA_ERR_MODE
    assert _fwd(lib, _desc(), odt=7) == _lib.BA_ERR_UNSUPPORTED
    assert _fwd(lib, _desc(causal=2)) == _lib.BA_ERR_SHAPE
    for bad_scale in (float("nan"), float("inf"), float("-inf")):
        d = _desc()
        d.scale = bad_scale
        assert _fwd(lib, d) == _lib.BA_ERR_SHAPE
        P = ctypes.c_void_p
        F = P(FAKE)
        assert lib.blockattn_bwd(ctypes.byref(d), F, F, F, F, F, F, F, F, F, F, 1, None, 0, None) == _lib.BA_ERR_SHAPE
        # the merge does not use the scale
        assert lib.lse_merge(ctypes.byref(d), F, F, P(FAKE + 4), 0, F, None, None) == _lib.BA_ERR_ALIGN


def test_zero_size_returns_ok_without_launch(lib):
    # nothing is enqueued (there is no GPU here: a launch would report BA_ERR_LAUNCH)
    assert _fwd(lib, _desc(B=0), q=0, k=0, v=0, o=0, lse=0) == _lib.BA_OK
    assert _fwd(lib, _desc(Sq=0), q=0, k=0, v=0, o=0, lse=0) == _lib.BA_OK


def test_merge_and_s2_validation(lib):
    P = ctypes.c_void_p
    d = _desc()
    assert lib.lse_merge(ctypes.byref(d), P(FAKE), P(FAKE), P(FAKE), 3, P(FAKE), None, None) == _lib.BA_ERR_UNSUPPORTED
    assert lib.lse_merge(ctypes.byref(d), P(FAKE), P(FAKE + 4), P(FAKE + 4), 0, P(FAKE), None, None) == _lib.BA_ERR_ALIGN
    assert lib.lse_merge(ctypes.byref(d), None, P(FAKE), P(FAKE), 0, P(FAKE), None, None) == _lib.BA_ERR_NULL

    def s2(desc, g, h0):
        s = _lib.BaS2Desc(g, h0)
        return lib.s2attn_fwd(ctypes.byref(desc), ctypes.byref(s), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 0,
                              P(FAKE), None)
    assert lib.s2attn_fwd(ctypes.byref(d), None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), 0, P(FAKE), None) == _lib.BA_ERR_NULL
    assert s2(_desc(Sq=1024, Sk=1024), 300, 1) == _lib.BA_ERR_S2       # group does not divide S
    assert s2(_desc(Sq=1024, Sk=1024), 128, 1) == _lib.BA_ERR_S2       # group/2 not a tile multiple
    assert s2(_desc(Sq=1024, Sk=1024), 256, 1) == _lib.BA_ERR_S2       # group/2 = 128: half a 256-row query tile
    assert s2(_desc(Sq=1024, Sk=512), 256, 1) == _lib.BA_ERR_S2        # Sq != Sk
    assert s2(_desc(Sq=1024, Sk=1024, k0=256), 256, 1) == _lib.BA_ERR_S2
    assert s2(_desc(Sq=1024, Sk=1024, Hq=8, Hkv=2), 256, 3) == _lib.BA_ERR_S2  # shift boundary inside a KV group
    assert s2(_desc(Sq=1024, Sk=1024), 256, 3) == _lib.BA_ERR_S2        # shift_head0 > Hq


def test_bwd_validation(lib):
    P = ctypes.c_void_p
    d = _desc(D=80)
    args = [P(FAKE)] * 10
    assert lib.blockattn_bwd(ctypes.byref(d), *args, 0, None, 0, None) == _lib.BA_ERR_UNSUPPORTED
    assert lib.blockattn_bwd(None, *args, 0, None, 0, None) == _lib.BA_ERR_NULL


# ---------------------------------------------------------------- tile schedule

def _covered_pairs(records, sq, sk):
    """Count how many times the schedule visits each (query row, key row) pair."""
    cnt = np.zeros((sq, sk), dtype=np.int64)
    for q0, qn, k0, kn in records:
        cnt[q0:q0 + qn, k0:k0 + kn] += 1
    return cnt


@pytest.mark.parametrize("kw", [
    dict(Sq=1000, Sk=1000),                      # ragged causal
    dict(Sq=512, Sk=256, k0=128),                # one ring chunk in the middle
    dict(Sq=512, Sk=100, k0=400),                # ragged last chunk
    dict(Sq=256, Sk=256, k0=512),                # chunk after every query: no work
    dict(Sq=300, Sk=200, q0=50, k0=0),           # query block offset
    dict(Sq=200, Sk=130, causal=0),              # non-causal
    dict(Sq=256, Sk=256, D=64),
])
def test_schedule_covers_allowed_pairs_once(lib, kw):
    d = _desc(**kw)
    rec = _lib.debug_fwd_schedule(d, head=0)
    cnt = _covered_pairs(rec, d.seqlen_q, d.seqlen_k)
    allowed = allowed_mask(d.q_pos0 + np.arange(d.seqlen_q), d.k_pos0 + np.arange(d.seqlen_k),
                           causal=bool(d.causal))
    assert cnt.max() <= 1, "a (query, key) pair is visited twice"
    assert np.all(cnt[allowed] == 1), "an allowed pair is never visited"
    # visited but disallowed pairs only occur inside diagonal tiles (masked in the kernel)
    bm, bn = _lib.debug_tile_sizes(d.head_dim)
    waste = cnt[~allowed].sum()
    assert waste <= d.seqlen_q * (bn + bm)


@pytest.mark.parametrize("shift_head0,head", [(2, 0), (2, 3), (0, 1)])
def test_schedule_s2(lib, shift_head0, head):
    S, G = 2048, 512
    d = _desc(Sq=S, Sk=S, Hq=4, Hkv=4)
    s2 = _lib.BaS2Desc(G, shift_head0)
    rec = _lib.debug_fwd_schedule(d, head=head, s2=s2)
    cnt = _covered_pairs(rec, S, S)
    allowed = allowed_mask(np.arange(S), np.arange(S), s2=S2Spec(G, shift_head0, S), head=head)
    assert cnt.max() <= 1
    assert np.all(cnt[allowed] == 1)
    # every visited pair lies in the same S2 group (cross-group pairs are never visited)
    same_group = allowed_mask(np.arange(S), np.arange(S), s2=S2Spec(G, shift_head0, S), head=head) | \
        allowed_mask(np.arange(S), np.arange(S), s2=S2Spec(G, shift_head0, S), head=head).T
    assert np.all(same_group[cnt > 0])


def test_schedule_longest_first(lib):
    d = _desc(Sq=1024, Sk=1024)
    rec = _lib.debug_fwd_schedule(d, head=0)
    # records come grouped by query tile in visiting order; tile work must not increase
    tiles = []
    for r in rec:
        if not tiles or tiles[-1][0] != r[0]:
            tiles.append([r[0], 0])
        tiles[-1][1] += 1
    work = [t[1] for t in tiles]
    assert work == sorted(work, reverse=True)


def test_ulysses_validation(lib):
    P = ctypes.c_void_p
    for fn in (lib.ulysses_pack, lib.ulysses_unpack):
        assert fn(P(FAKE), P(FAKE), 1, 16, 30, 128, 8, None) == _lib.BA_ERR_SHAPE    # heads % N
        assert fn(P(FAKE), P(FAKE), 1, 16, 32, 128, 0, None) == _lib.BA_ERR_SHAPE    # N < 1
        assert fn(P(FAKE), P(FAKE), 1, 16, 32, 100, 8, None) == _lib.BA_ERR_SHAPE    # D % 8
        assert fn(P(FAKE), P(FAKE), -1, 16, 32, 128, 8, None) == _lib.BA_ERR_SHAPE
        assert fn(None, P(FAKE), 1, 16, 32, 128, 8, None) == _lib.BA_ERR_NULL
        assert fn(P(FAKE), P(FAKE + 8), 1, 16, 32, 128, 8, None) == _lib.BA_ERR_ALIGN
        assert fn(None, None, 1, 0, 32, 128, 8, None) == _lib.BA_OK                  # zero size, no launch


def test_bpt_ffn_validation(lib):
    P = ctypes.c_void_p
    args = [P(FAKE)] * 6
    assert lib.bpt_ffn(*args, 100, 300, 256, 64, None) == _lib.BA_ERR_SHAPE     # d_model % 256
    assert lib.bpt_ffn(*args, 100, 256, 200, 64, None) == _lib.BA_ERR_SHAPE     # d_ff % 128
    assert lib.bpt_ffn(*args, 100, 256, 256, 0, None) == _lib.BA_ERR_SHAPE      # block_rows
    assert lib.bpt_ffn(*args, 1 << 24, 256, 256, 64, None) == _lib.BA_ERR_SHAPE  # 2^32 elements of x
    assert lib.bpt_ffn(None, *args[1:], 100, 256, 256, 64, None) == _lib.BA_ERR_NULL
    assert lib.bpt_ffn(P(FAKE + 2), *args[1:], 100, 256, 256, 64, None) == _lib.BA_ERR_ALIGN
    assert lib.bpt_ffn(None, None, None, None, None, None, 0, 256, 256, 64, None) == _lib.BA_OK


class _FakeGpuTensor:
    """Stands in for a GPU tensor in the binding's checks (no data, never passed on)."""

    def __init__(self, dtype, device="cuda:0"):
        import torch
        self.is_cuda = True
        self.device = torch.device(device)
        self.dtype = dtype


def test_binding_rejects_host_tensors_before_any_call():
    import torch
    q = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError, match="GPU"):
        _lib.blockattn_fwd(q, q, q, q.float(), lse)
    with pytest.raises(ValueError, match="GPU"):
        _lib.lse_merge(q.float(), lse, q.float(), lse)
    with pytest.raises(ValueError, match="GPU"):
        _lib.blockattn_bwd(q, q, q, q, q, lse, lse, q.float(), q, q)
    with pytest.raises(ValueError, match="GPU"):
        _lib.s2attn_fwd(q, q, q, q.float(), lse, group=64, shift_head0=2)
    with pytest.raises(ValueError, match="GPU"):
        _lib.ulysses_pack(q, 2)
    with pytest.raises(ValueError, match="GPU"):
        _lib.bpt_ffn(q[0, :, 0], q[0, :, 0], q[0, :, 0], q[0, :, 0])


def test_binding_dtype_and_device_requirements():
    import torch
    q = _FakeGpuTensor(torch.bfloat16)
    _lib._require(q, [(q, "q", "bfloat16"), (_FakeGpuTensor(torch.float32), "lse", "float32"), (None, "x", "float32")])
    # a bf16 statistics tensor would be written with fp32 stores past its end
    with pytest.raises(ValueError, match="lse must be float32"):
        _lib._require(q, [(_FakeGpuTensor(torch.bfloat16), "lse", "float32")])
    with pytest.raises(ValueError, match="k must be bfloat16"):
        _lib._require(q, [(_FakeGpuTensor(torch.float32), "k", "bfloat16")])
    with pytest.raises(ValueError, match="must be on cuda:0"):
        _lib._require(q, [(_FakeGpuTensor(torch.bfloat16, "cuda:1"), "v", "bfloat16")])


def test_ring_drivers_reject_bad_chunk_orders():
    import torch
    from long_context_exact_blockattn_amd import ring_backward, ring_forward
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 64)
    for bad in ([0, 0, 1, 2], [0, 1, 2], [1, 2, 3, 4]):
        with pytest.raises(ValueError, match="permutation"):
            ring_forward(q, q, q, 4, bad)
        with pytest.raises(ValueError, match="permutation"):
            ring_backward(q, q, q, q, q, lse, 4, bad)


@pytest.mark.parametrize("Sq,Sk,q0,k0", [(1000, 250, 0, 750), (1000, 250, 0, 130), (512, 64, 0, 512),
                                         (300, 100, 50, 280), (2048, 512, 0, 1536), (256, 100, 300, 0)])
def test_unreached_causal_tiles_are_the_last_ranks(lib, Sq, Sk, q0, k0):
    # an ACCUMULATE ring step launches only the first (n_qtiles - skip) ranks, skip = the query
    # tiles wholly before the chunk; this needs those tiles to have no key tile to visit and
    # to come last in the visiting order
    d = _desc(Sq=Sq, Sk=Sk, q0=q0, k0=k0)
    bm, _ = _lib.debug_tile_sizes(d.head_dim)
    skip = min(max(k0 - q0, 0), Sq) // bm
    rec = _lib.debug_fwd_schedule(d, head=0)
    visited = [int(r) for r in dict.fromkeys(rec[:, 0])]  # query tiles' first rows, visiting order
    assert all(r >= skip * bm for r in visited), "a skipped tile has work"
    n_qtiles = -(-Sq // bm)
    launched = sorted(range(skip, n_qtiles), reverse=True)  # ranks 0 .. n_qtiles - skip - 1
    assert [r // bm for r in visited] == launched[:len(visited)]


def test_binding_layout_check_ignores_length_one_axes():
    """The kernels address the tensors of one stride group with one set of strides; an axis of
    length one is never stepped along, so its stride may differ (torch keeps a slice's batch
    stride in .contiguous() of a batch of one), while a real stride mismatch is refused."""
    import torch
    o = torch.zeros(1, 1000, 4, 128)[:, 300:700].contiguous()
    dout = torch.zeros(1, 400, 4, 128)
    assert o.stride(0) != dout.stride(0)
    _lib._same_layout(o, dout, "dout")
    o2 = torch.zeros(2, 1000, 4, 128)[:, 300:700]
    with pytest.raises(ValueError, match="strides as o"):
        _lib._same_layout(o2, torch.zeros(2, 400, 4, 128), "dout")
    k = torch.zeros(2, 64, 1, 128)
    v = torch.zeros(2, 64, 3, 128)[:, :, 1:2]  # sequence stride 384 against k's 128
    with pytest.raises(ValueError, match="strides as k"):
        _lib._same_layout(k, v, "v", ref_name="k")
    # one head: only the (unused) head stride differs
    v1 = torch.zeros(2 * 64 * 128 + 1000).as_strided((2, 64, 1, 128), (8192, 128, 999, 1))
    _lib._same_layout(k, v1, "v", ref_name="k")


def test_descriptor_zeroes_strides_of_length_one_axes(lib):
    """A batch of one sliced at an odd element offset has an odd batch stride that no kernel ever
    uses; the descriptor carries 0 there, so the call passes the library's stride rules."""
    import torch
    x = torch.zeros(1, 300, 2, 128).as_strided((1, 300, 2, 128), (12345, 256, 128, 1))
    d = _lib.make_desc(x, x)
    assert tuple(d.q_stride) == (0, 256, 128) and tuple(d.kv_stride) == (0, 256, 128)
    assert tuple(d.o_stride) == (0, 256, 128)
    # validation passes the strides and stops at the (fake) misaligned pointer instead
    assert _fwd(lib, d, q=FAKE + 2) == _lib.BA_ERR_ALIGN
    y = torch.zeros(2, 1, 2, 128)
    assert tuple(_lib.make_desc(y, y).q_stride) == (256, 0, 128)


def test_descriptor_refuses_k_of_another_batch_or_head_size():
    """The descriptor holds one batch size and one head size: a k that differs in either would be
    read past its end (or, with a batch of one, silently reused), so the binding refuses it."""
    import torch
    q = torch.zeros(2, 64, 4, 128)
    with pytest.raises(ValueError, match="batch"):
        _lib.make_desc(q, torch.zeros(1, 64, 2, 128))
    with pytest.raises(ValueError, match="head_dim"):
        _lib.make_desc(q, torch.zeros(2, 64, 2, 64))
    with pytest.raises(ValueError, match=r"\[B, S, H, D\]"):
        _lib.make_desc(q, torch.zeros(2, 64, 128))
    d = _lib.make_desc(q, torch.zeros(2, 32, 2, 128))  # other length and head count: the ABI's business
    assert (d.batch, d.heads_q, d.heads_kv, d.seqlen_q, d.seqlen_k) == (2, 4, 2, 64, 32)


def test_descriptor_output_strides_independent_of_q():
    """q may be a strided view (a slice of a packed [B, S, 3, H, D] projection) while the outputs
    are dense: q_stride comes from q, o_stride from o, kv_stride from k."""
    import torch
    B, S, H, D = 2, 64, 4, 128
    packed = torch.zeros(B, S, 3, H, D)
    q, k = packed[:, :, 0], packed[:, :, 1]
    o = torch.zeros(B, S, H, D)
    d = _lib.make_desc(q, k, o)
    assert tuple(d.q_stride) == (S * 3 * H * D, 3 * H * D, D)
    assert tuple(d.kv_stride) == (S * 3 * H * D, 3 * H * D, D)
    assert tuple(d.o_stride) == (S * H * D, H * D, D)
    assert tuple(_lib.make_desc(q, k).o_stride) == tuple(d.q_stride)  # no o: q's own strides
    with pytest.raises(ValueError, match="shape"):
        _lib.make_desc(q, k, torch.zeros(B, S + 1, H, D))


def test_noalloc_rejects_problems_beyond_its_scratch_buffer(lib):
    """blockattn_bwd_noalloc checks the problem against its static buffer before anything else
    touches the GPU (so this runs without one)."""
    P = ctypes.c_void_p
    d = _desc(B=1, Hq=64, Hkv=8, Sq=(1 << 17) + 1, Sk=256)
    st = lib.blockattn_bwd_noalloc(ctypes.byref(d), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                   P(FAKE), P(FAKE), P(FAKE), _lib.BA_BF16, None, 0, None)
    assert st == _lib.BA_ERR_WORKSPACE
    assert "scratch" in _lib.status_string(st)
    assert lib.blockattn_bwd_noalloc(None, *([P(FAKE)] * 9), _lib.BA_BF16, None, 0, None) == _lib.BA_ERR_NULL
    d = _desc(Sq=-1)
    assert lib.blockattn_bwd_noalloc(ctypes.byref(d), *([P(FAKE)] * 9), _lib.BA_BF16, None, 0, None) == _lib.BA_ERR_SHAPE


def test_final_store_steps_cover_every_rows_last_reaching_step():
    """Under the causal mask chunk c reaches the row blocks c, c+1, ...; the positions that store
    the final output (ring.final_store_steps) must include every block's last reaching position,
    and a stored value is final only there: brute force over all orders of up to 6 chunks and
    random orders of 16."""
    import itertools
    import random
    from long_context_exact_blockattn_amd.ring import final_store_steps
    orders = [list(p) for n in range(1, 7) for p in itertools.permutations(range(n))]
    rnd = random.Random(0)
    orders += [rnd.sample(range(16), 16) for _ in range(200)]
    for order in orders:
        n = len(order)
        store = final_store_steps(order)
        assert store[-1]
        for blk in range(n):
            reaching = [t for t, c in enumerate(order) if c <= blk]
            writes = [t for t in reaching if store[t]]  # stores touch only rows their chunk reaches
            assert writes and writes[-1] == reaching[-1], (order, blk)
        assert final_store_steps(order, causal=False) == [t == n - 1 for t in range(n)]
    # the headline order stores at three positions: chunks 0 (block 0), 1 (blocks 1-6), 7 (block 7)
    assert final_store_steps([2, 4, 3, 6, 5, 0, 1, 7]) == [False] * 5 + [True] * 3
