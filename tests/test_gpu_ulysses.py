"""GPU parity of the Ulysses layout permutes (bit-exact against oracle/ulysses.py) and of the
emulated Ulysses forward: N devices' shards packed, exchanged (emulated by indexing on one GPU),
attention over the whole sequence of each head group, equal bit for bit to the head slices of the
same kernels run on all heads at once (heads are independent)."""
import numpy as np
import pytest
import torch

import long_context_exact_blockattn_amd as ba
from oracle import attention_forward
from oracle.ulysses import pack, unpack
from tests.gpu_helpers import TOL_LSE, TOL_O, dev, f64, log, max_err
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("B,Sl,H,D,N", [(1, 4096, 32, 128, 8), (2, 1000, 8, 64, 4), (1, 37, 4, 128, 1),
                                        (1, 513, 40, 128, 8)])
def test_pack_unpack_bit_exact(B, Sl, H, D, N):
    g = torch.Generator().manual_seed(Sl + N)
    x = torch.randn(B, Sl, H, D, generator=g).to(torch.bfloat16)
    send = ba.ulysses_pack(x.to(dev()), N)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(send), pack(_bits(x), N))
    back = ba.ulysses_unpack(send, N)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(back), unpack(pack(_bits(x), N), N))
    assert torch.equal(back.cpu(), x)


def test_emulated_ulysses_forward_matches_full_heads():
    B, N, S, H, D = 1, 4, 2048, 8, 128
    Sl, hn = S // N, H // N
    q, k, v = make_inputs(B, S, H, H, D, seed=70)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    # each device packs its sequence shard; the exchange hands device n block n of every shard
    sends = {name: [ba.ulysses_pack(t[:, r * Sl:(r + 1) * Sl].contiguous(), N) for r in range(N)]
             for name, t in (("q", qd), ("k", kd), ("v", vd))}
    full_out, full_lse, _ = ba.ring_forward(qd, kd, vd, 1)
    outs = []
    for n in range(N):
        qn, kn, vn = (torch.cat([sends[name][r][n] for r in range(N)], dim=1) for name in ("q", "k", "v"))
        o, lse, _ = ba.ring_forward(qn, kn, vn, 1)
        assert torch.equal(o, full_out[:, :, n * hn:(n + 1) * hn])
        assert torch.equal(lse, full_lse[:, n * hn:(n + 1) * hn])
        outs.append(o)
    # back: device n's output rows of chunk r go to device r, which unpacks its rows of all heads
    for r in range(N):
        recv = torch.stack([outs[n][:, r * Sl:(r + 1) * Sl] for n in range(N)]).contiguous()
        assert torch.equal(ba.ulysses_unpack(recv, N), full_out[:, r * Sl:(r + 1) * Sl])
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_forward(f64(q), f64(k), f64(v))
    err = max_err(full_out, o_ref)
    log(f"emulated Ulysses N={N}: equal to the all-heads run; that run vs oracle: O {err:.3e}")
    assert err <= TOL_O and max_err(full_lse, lse_ref) <= TOL_LSE
