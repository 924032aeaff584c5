"""Pins of the Ulysses layout oracle (oracle/ulysses.py) against what the method fixes.

- A hand-worked example (N=2, H=4): the values of every send block written out.
- Round trip: unpack(pack(x)) == x.
- The defining property of the exchange: with X split into N sequence shards, each packed, and the
  all-to-all applied, device n ends up with all S rows of head group n, i.e. X[:, :, group n].
- Its use around attention: attention over the whole sequence of a head group, computed from the
  received blocks, equals the head group's slice of attention over all heads (heads are independent).
"""
import numpy as np
import pytest

from oracle import attention_forward
from oracle.ulysses import alltoall, gather_sequence, pack, unpack


def test_handworked_example():
    # x[0, s, h, 0] = 10 s + h, Sl = 2, H = 4, D = 1, N = 2 (head groups {0,1}, {2,3})
    x = np.array([[[[0], [1], [2], [3]], [[10], [11], [12], [13]]]], dtype=np.int64)
    send = pack(x, 2)
    assert send.shape == (2, 1, 2, 2, 1)
    assert send[0, 0, :, :, 0].tolist() == [[0, 1], [10, 11]]
    assert send[1, 0, :, :, 0].tolist() == [[2, 3], [12, 13]]
    assert unpack(send, 2).tolist() == x.tolist()


@pytest.mark.parametrize("B,Sl,H,D,N", [(1, 5, 8, 3, 4), (2, 3, 6, 2, 3), (1, 4, 4, 1, 1)])
def test_round_trip(B, Sl, H, D, N):
    x = np.random.default_rng(0).standard_normal((B, Sl, H, D))
    assert np.array_equal(unpack(pack(x, N), N), x)


@pytest.mark.parametrize("B,N,Sl,H,D", [(1, 4, 3, 8, 2), (2, 2, 5, 6, 3)])
def test_exchange_gives_each_device_its_heads_over_the_whole_sequence(B, N, Sl, H, D):
    X = np.random.default_rng(1).standard_normal((B, N * Sl, H, D))
    shards = [X[:, r * Sl:(r + 1) * Sl] for r in range(N)]
    recvs = alltoall([pack(x, N) for x in shards])
    hn = H // N
    for n in range(N):
        assert np.array_equal(gather_sequence(recvs[n]), X[:, :, n * hn:(n + 1) * hn])
    # and back: the same exchange of the per-device results, unpacked, restores the shards
    back = alltoall([np.stack([r[m] for m in range(N)]) for r in recvs])
    for r in range(N):
        assert np.array_equal(unpack(back[r], N), shards[r])


def test_attention_on_received_blocks_equals_head_slice_of_full_attention():
    rng = np.random.default_rng(2)
    B, N, Sl, H, D = 1, 4, 6, 8, 4
    Q, K, V = (rng.standard_normal((B, N * Sl, H, D)) for _ in range(3))
    o_full, lse_full = attention_forward(Q, K, V)
    hn = H // N
    for n in range(N):
        q, k, v = (gather_sequence(alltoall([pack(T[:, r * Sl:(r + 1) * Sl], N) for r in range(N)])[n])
                   for T in (Q, K, V))
        o, lse = attention_forward(q, k, v)
        assert np.allclose(o, o_full[:, :, n * hn:(n + 1) * hn], atol=1e-13)
        assert np.allclose(lse, lse_full[:, n * hn:(n + 1) * hn], atol=1e-13)
