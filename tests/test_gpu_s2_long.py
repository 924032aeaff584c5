"""S2-Attn at long context (S=102400, group 25600 = S/4, heads 16-31 shifted by 12800), forward and
backward of all 32 heads on the GPU, checked against the oracle on what it can compute at this size:

- O, LSE and dQ of sampled rows of an unshifted and a shifted head (every group edge, the wrap
  group of the shifted heads, seeded random rows), from the oracle's single-row definitions;
- dQ, dK, dV of one whole group of an unshifted and of a shifted head: a group only attends within
  itself (causally, in rolled order), so the group's slice of the original sequence -- contiguous,
  starting G/2 later for a shifted head -- is plain causal attention, and the oracle's full backward
  of that slice is the exact gradient there.
Gates as elsewhere: O 1e-2, LSE 1e-3 absolute; gradients relative L2 2e-2.
"""
import numpy as np
import pytest
import torch

import long_context_exact_blockattn_amd as ba
from oracle import S2Spec, attention_backward, rows_backward_dq, rows_forward
from tests.gpu_helpers import TOL_GRAD, TOL_LSE, TOL_O, dev, f64, log, max_err, rel_l2
from workloads import get, make_inputs

pytestmark = pytest.mark.gpu


def test_s2_long_context_fwd_bwd():
    w = get("s2attn_llama2_7b_s100k_g25600")
    S, G, H = w.seqlen, w.s2_group, w.heads_q
    log("S2 long: generating inputs")
    q, k, v, do = make_inputs(w.batch, S, H, w.heads_kv, w.head_dim, seed=w.seed, with_dout=True)
    qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
    o, lse = ba.s2_forward(qd, kd, vd, G, w.s2_shift_head0)
    dq, dk, dv = ba.s2_backward(qd, kd, vd, o, dod, lse, G, w.s2_shift_head0)
    torch.cuda.synchronize()
    spec = S2Spec(G, w.s2_shift_head0, S)
    qn, kn, vn, don = (t.float().numpy() for t in (q, k, v, do))
    rng = np.random.default_rng(5)
    edges = {0, 1, G // 2 - 1, G // 2, G - 1, G, 2 * G - 1, S - G // 2 - 1, S - G // 2, S - 1}
    rows = sorted(edges | set(map(int, rng.integers(0, S, 10))))
    for h in (3, 16 + 5):
        o_ref, lse_ref = rows_forward(qn, kn, vn, 0, h, rows, s2=spec)
        eo = max_err(o[0, rows, h].float().cpu(), o_ref)
        el = max_err(lse[0, h, rows].cpu(), lse_ref)
        dq_ref = rows_backward_dq(qn, kn, vn, don, 0, h, rows, s2=spec)
        eq = rel_l2(dq[0, rows, h].float().cpu(), dq_ref)
        log(f"S2 long head {h}: sampled rows O {eo:.3e} LSE {el:.3e} dQ rel {eq:.3e}")
        assert eo <= TOL_O and el <= TOL_LSE and eq <= TOL_GRAD
    # whole groups: unshifted head 3, group 1; shifted head 21, group 1 (original rows G/2 + G ...)
    for h, start in ((3, G), (16 + 5, G // 2 + G)):
        sl = slice(start, start + G)
        sub = [np.ascontiguousarray(t[:, sl, h:h + 1]) for t in (qn, kn, vn, don)]
        log(f"S2 long head {h}: oracle backward of the group at rows {start}..{start + G - 1}")
        gq, gk, gv, _, _ = attention_backward(*sub, row_block=2048)
        got = [t[:, sl, h:h + 1].float().cpu() for t in (dq, dk, dv)]
        errs = [rel_l2(g, r) for g, r in zip(got, (gq, gk, gv))]
        log(f"S2 long head {h} group: rel L2 dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}")
        assert max(errs) <= TOL_GRAD
