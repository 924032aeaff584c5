"""Pins for the CPU oracle: checks against things other than the oracle itself.

Hand-derived golden values, pure-loop brute force on tiny inputs, closed forms,
library routines (torch's fp64 scaled_dot_product_attention and autograd),
finite differences and exact identities.  A dropped term, a wrong sign, a
transposed operand or a wrong mask convention in the oracle fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (NEG_INF, S2Spec, allowed_mask, attention_backward, attention_forward,
                    backward_delta, default_scale, lse_merge, ring_attention_forward, rows_forward)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _expr(s):
    return float(eval(s, {"log": math.log, "inf": math.inf}))


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- golden values

def test_golden_forward_handworked():
    g = _load("handworked_forward.json")
    q = np.array(g["q"]).reshape(1, 3, 1, 1)
    k = np.array(g["k"]).reshape(1, 3, 1, 1)
    v = np.array(g["v"]).reshape(1, 3, 1, 1)
    o, lse = attention_forward(q, k, v, scale=g["scale"], causal=True)
    np.testing.assert_allclose(o[0, :, 0, 0], g["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], [_expr(e) for e in g["lse_exprs"]], rtol=0, atol=1e-13)


def test_golden_merge_handworked():
    g = _load("handworked_merge.json")
    for c in g["cases"]:
        oa = np.full((1, 1, 1, 1), c["o_a"])
        ob = np.full((1, 1, 1, 1), c["o_b"])
        la = np.full((1, 1, 1), _expr(c["lse_a"]))
        lb = np.full((1, 1, 1), _expr(c["lse_b"]))
        o, l = lse_merge(oa, la, ob, lb)
        assert o[0, 0, 0, 0] == pytest.approx(c["o"], abs=1e-13)
        want = _expr(c["lse"])
        if math.isinf(want):
            assert l[0, 0, 0] == -math.inf
        else:
            assert l[0, 0, 0] == pytest.approx(want, abs=1e-13)


def test_golden_backward_handworked():
    g = _load("handworked_backward.json")
    sh = (1, 2, 1, 1)
    q, k, v, do = (np.array(g[n]).reshape(sh) for n in ("q", "k", "v", "dout"))
    dq, dk, dv, o, _ = attention_backward(q, k, v, do, scale=g["scale"], causal=True)
    np.testing.assert_allclose(o.ravel(), g["o"], atol=1e-13)
    np.testing.assert_allclose(dq.ravel(), g["dq"], atol=1e-13)
    np.testing.assert_allclose(dk.ravel(), [_expr(e) for e in g["dk_exprs"]], atol=1e-13)
    np.testing.assert_allclose(dv.ravel(), g["dv"], atol=1e-13)


def test_golden_backward_delta_handworked():
    # Delta of the hand-worked example, from the hand-derived O and from the oracle's own O
    g = _load("handworked_backward.json")
    sh = (1, 2, 1, 1)
    o, do = (np.array(g[n]).reshape(sh) for n in ("o", "dout"))
    np.testing.assert_allclose(backward_delta(o, do).ravel(), g["delta"], atol=1e-13)
    q, k, v = (np.array(g[n]).reshape(sh) for n in ("q", "k", "v"))
    o_or, _ = attention_forward(q, k, v, scale=g["scale"], causal=True)
    np.testing.assert_allclose(backward_delta(o_or, do).ravel(), g["delta"], atol=1e-13)


def test_golden_s2_allowed_sets():
    g = _load("s2_allowed_sets.json")
    s, grp = g["seqlen"], g["group"]
    spec = S2Spec(group=grp, shift_head0=1, seqlen=s)
    pos = np.arange(s)
    for head, key in ((0, "unshifted"), (1, "shifted")):
        m = allowed_mask(pos, pos, s2=spec, head=head)
        for i in range(s):
            assert sorted(np.nonzero(m[i])[0].tolist()) == sorted(g[key][str(i)]), (key, i)


# ---------------------------------------------------------------- brute force

def _brute_forward(q, k, v, scale, allowed):
    """Triple loop with math.exp; allowed(b, h, i, j) -> bool."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    o = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Hq, Sq), -math.inf)
    for b in range(B):
        for h in range(Hq):
            kh = h // grp
            for i in range(Sq):
                scores = []
                for j in range(Sk):
                    if allowed(b, h, i, j):
                        dot = 0.0
                        for d in range(D):
                            dot += q[b, i, h, d] * k[b, j, kh, d]
                        scores.append((j, scale * dot))
                if not scores:
                    continue
                mx = max(s for _, s in scores)
                z = sum(math.exp(s - mx) for _, s in scores)
                lse[b, h, i] = mx + math.log(z)
                for j, s in scores:
                    w = math.exp(s - mx) / z
                    for d in range(D):
                        o[b, i, h, d] += w * v[b, j, kh, d]
    return o, lse


@pytest.mark.parametrize("case", [
    dict(B=1, Sq=9, Sk=9, Hq=2, Hkv=2, D=4, causal=True, q0=0, k0=0),
    dict(B=2, Sq=7, Sk=5, Hq=4, Hkv=2, D=3, causal=True, q0=3, k0=2),
    dict(B=1, Sq=6, Sk=4, Hq=2, Hkv=1, D=5, causal=True, q0=0, k0=4),   # rows with no key
    dict(B=1, Sq=5, Sk=6, Hq=3, Hkv=3, D=2, causal=False, q0=0, k0=0),
])
def test_bruteforce_forward(case):
    c = case
    q = _rand((c["B"], c["Sq"], c["Hq"], c["D"]), 1)
    k = _rand((c["B"], c["Sk"], c["Hkv"], c["D"]), 2)
    v = _rand((c["B"], c["Sk"], c["Hkv"], c["D"]), 3)
    tau = 1.0 / math.sqrt(c["D"])

    def allowed(b, h, i, j):
        return (not c["causal"]) or (c["k0"] + j <= c["q0"] + i)

    ob, lb = _brute_forward(q, k, v, tau, allowed)
    o, l = attention_forward(q, k, v, causal=c["causal"], q_pos0=c["q0"], k_pos0=c["k0"])
    np.testing.assert_allclose(o, ob, atol=1e-12)
    assert np.array_equal(np.isinf(l), np.isinf(lb))
    np.testing.assert_allclose(l[np.isfinite(l)], lb[np.isfinite(lb)], atol=1e-12)


def _brute_delta_by_probs(q, k, v, do, scale, allowed):
    """Delta[b, h, i] as sum_j P_ij dP_ij, every quantity by plain loops: P from the scores,
    dP_ij = dO_i . V_j.  Since sum_j P_ij V_j = O_i this equals dO_i . O_i, but it is built
    without forming O, so a Delta taken from the wrong row, head or batch does not match."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    delta = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            kh = h // grp
            for i in range(Sq):
                js = [j for j in range(Sk) if allowed(b, h, i, j)]
                if not js:
                    continue
                s = {j: scale * sum(q[b, i, h, d] * k[b, j, kh, d] for d in range(D)) for j in js}
                mx = max(s.values())
                z = sum(math.exp(x - mx) for x in s.values())
                for j in js:
                    p = math.exp(s[j] - mx) / z
                    dp = sum(do[b, i, h, d] * v[b, j, kh, d] for d in range(D))
                    delta[b, h, i] += p * dp
    return delta


def _check_backward_delta(fn):
    """Pin of backward_delta (or a stand-in fn with its signature): on B=2, S=6, Hq=4, Hkv=2,
    D=3 (every axis a different length, so a wrong axis order cannot pass) it must equal the
    pure-loop sum_j P_ij dP_ij, with the O it is given being the pure-loop forward's O."""
    B, S, Hq, Hkv, D = 2, 6, 4, 2, 3
    q = _rand((B, S, Hq, D), 160)
    k = _rand((B, S, Hkv, D), 161)
    v = _rand((B, S, Hkv, D), 162)
    do = _rand((B, S, Hq, D), 163)
    tau = 1.0 / math.sqrt(D)
    allowed = lambda b, h, i, j: j <= i
    o_bf, _ = _brute_forward(q, k, v, tau, allowed)
    want = _brute_delta_by_probs(q, k, v, do, tau, allowed)
    got = fn(o_bf, do)
    assert got.shape == want.shape, (got.shape, want.shape)
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_bruteforce_backward_delta():
    _check_backward_delta(backward_delta)


def test_bruteforce_forward_s2():
    S, G, H, D = 12, 4, 4, 3
    q, k, v = (_rand((1, S, H, D), s) for s in (4, 5, 6))
    spec = S2Spec(group=G, shift_head0=2, seqlen=S)

    def allowed(b, h, i, j):
        # groups listed explicitly in original positions, built by walking the rolled order
        sh = G // 2 if h >= 2 else 0
        order = [(r + sh) % S for r in range(S)]          # rolled slot r holds original order[r]
        slot = {p: r for r, p in enumerate(order)}
        return slot[i] // G == slot[j] // G and slot[j] <= slot[i]

    ob, lb = _brute_forward(q, k, v, 1.0 / math.sqrt(D), allowed)
    o, l = attention_forward(q, k, v, s2=spec)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(l, lb, atol=1e-12)


def test_rows_forward_matches_full():
    q, k, v = (_rand((2, 40, 4, 8), s) for s in (7, 8, 9))
    k2, v2 = k[:, :, :2], v[:, :, :2]
    o, l = attention_forward(q, k2, v2)
    rows = [0, 5, 39, 17]
    for b in range(2):
        for h in range(4):
            orow, lrow = rows_forward(q, k2, v2, b, h, rows)
            np.testing.assert_allclose(orow, o[b, rows, h], atol=1e-14)
            np.testing.assert_allclose(lrow, l[b, h, rows], atol=1e-14)


# ---------------------------------------------------------------- closed forms

def test_closed_form_zero_queries():
    """Q = 0: every allowed score is 0, so O_i is the mean of V_0..V_i and LSE_i = ln(i+1)."""
    S, H, D = 33, 2, 6
    q = np.zeros((1, S, H, D))
    k = _rand((1, S, H, D), 11)
    v = _rand((1, S, H, D), 12)
    o, l = attention_forward(q, k, v)
    means = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    np.testing.assert_allclose(o, means, atol=1e-13)
    np.testing.assert_allclose(l, np.broadcast_to(np.log(np.arange(1, S + 1)), l.shape), atol=1e-13)


def test_closed_form_first_row():
    q, k, v = (_rand((1, 10, 3, 8), s) for s in (13, 14, 15))
    o, l = attention_forward(q, k, v)
    np.testing.assert_allclose(o[0, 0], v[0, 0], atol=1e-14)
    tau = default_scale(8)
    np.testing.assert_allclose(l[0, :, 0], tau * np.sum(q[0, 0] * k[0, 0], axis=-1), atol=1e-14)


def test_key_shift_invariance():
    """Adding w to every key adds tau q_i.w to every score of row i: O unchanged, LSE shifted."""
    q, k, v = (_rand((1, 20, 2, 8), s) for s in (16, 17, 18))
    w = _rand((8,), 19)
    o1, l1 = attention_forward(q, k, v)
    o2, l2 = attention_forward(q, k + w, v)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    tau = default_scale(8)
    np.testing.assert_allclose(l2 - l1, tau * np.einsum("bshd,d->bhs", q, w), atol=1e-12)


def test_torch_sdpa_fp64():
    """Library routine: torch's causal scaled_dot_product_attention in float64 on the CPU."""
    B, S, H, D = 2, 70, 3, 16
    q, k, v = (_rand((B, S, H, D), s) for s in (20, 21, 22))
    o, _ = attention_forward(q, k, v)
    t = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


# ---------------------------------------------------------------- ring / merge

@pytest.mark.parametrize("n_chunks,sk", [(4, 64), (5, 61), (3, 9)])
def test_ring_order_independence(n_chunks, sk):
    q, k, v = (_rand((1, sk, 2, 8), s) for s in (23, 24, 25))
    o_ref, l_ref = attention_forward(q, k, v)
    clen = -(-sk // n_chunks)
    for seed in range(4):
        order = np.random.default_rng(seed).permutation(n_chunks)
        o, l = ring_attention_forward(q, k, v, order, clen)
        np.testing.assert_allclose(o, o_ref, atol=1e-13)
        np.testing.assert_allclose(l, l_ref, atol=1e-13)


def test_single_chunk_is_one_shot():
    q, k, v = (_rand((1, 30, 2, 8), s) for s in (26, 27, 28))
    o_ref, l_ref = attention_forward(q, k, v)
    o, l = ring_attention_forward(q, k, v, [0], 30)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(l, l_ref)


def test_merge_algebra():
    sh_o, sh_l = (1, 6, 2, 4), (1, 2, 6)
    pairs = [(_rand(sh_o, 30 + i), _rand(sh_l, 40 + i)) for i in range(3)]
    pairs[1][1][0, 0, 2] = -np.inf         # an empty partial row
    a, b, c = pairs
    ab = lse_merge(*a, *b)
    ba = lse_merge(*b, *a)
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-14)
    np.testing.assert_allclose(ab[1], ba[1], atol=1e-14)
    left = lse_merge(*ab, *c)
    right = lse_merge(*a, *lse_merge(*b, *c))
    np.testing.assert_allclose(left[0], right[0], atol=1e-13)
    np.testing.assert_allclose(left[1], right[1], atol=1e-13)
    ident = (np.full(sh_o, np.nan), np.full(sh_l, -np.inf))   # O of an empty pair is ignored
    o, l = lse_merge(*a, *ident)
    np.testing.assert_array_equal(o, a[0])
    np.testing.assert_array_equal(l, a[1])


def test_merge_equals_one_shot_split_keys():
    """Merging the partials over two disjoint key sets equals attention over their union."""
    q, k, v = (_rand((1, 16, 2, 8), s) for s in (50, 51, 52))
    o_ref, l_ref = attention_forward(q, k, v, causal=False)
    oa, la = attention_forward(q, k[:, :5], v[:, :5], causal=False)
    ob, lb = attention_forward(q, k[:, 5:], v[:, 5:], causal=False, k_pos0=5)
    o, l = lse_merge(oa, la, ob, lb)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, atol=1e-13)


# ---------------------------------------------------------------- backward

def _torch_attention(q, k, v, scale, mask):
    """Plain torch ops (float64) for autograd: softmax over masked scores, per KV-head mapping."""
    hq, hkv = q.shape[2], k.shape[2]
    kk = k.repeat_interleave(hq // hkv, dim=2)
    vv = v.repeat_interleave(hq // hkv, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", q, kk) * scale
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.einsum("bhij,bjhd->bihd", p, vv)


@pytest.mark.parametrize("hq,hkv,s2", [(2, 2, None), (4, 2, None), (4, 4, S2Spec(8, 2, 24))])
def test_backward_vs_autograd(hq, hkv, s2):
    S, D = 24, 8
    q, k, v, do = (_rand((1, S, h, D), s) for h, s in ((hq, 60), (hkv, 61), (hkv, 62), (hq, 63)))
    dq, dk, dv, o, _ = attention_backward(q, k, v, do, s2=s2)
    tq, tk, tv = (torch.from_numpy(a).requires_grad_() for a in (q, k, v))
    pos = np.arange(S)
    mask = torch.stack([torch.from_numpy(allowed_mask(pos, pos, s2=s2, head=h)) for h in range(hq)])[None]
    out = _torch_attention(tq, tk, tv, default_scale(D), mask)
    np.testing.assert_allclose(out.detach().numpy(), o, atol=1e-13)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_backward_finite_differences():
    S, H, D = 7, 2, 3
    q, k, v, do = (_rand((1, S, H, D), s) for s in (70, 71, 72, 73))
    dq, dk, dv, _, _ = attention_backward(q, k, v, do)
    f = lambda qq, kk, vv: float(np.sum(attention_forward(qq, kk, vv)[0] * do))
    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = plus, minus
            num = (f(args_p["q"], args_p["k"], args_p["v"]) - f(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            assert grad[idx] == pytest.approx(num, abs=1e-7), (name, idx)


@pytest.mark.parametrize("hq,hkv,s2", [(2, 2, None), (4, 1, None), (4, 4, S2Spec(8, 2, 32))])
def test_backward_identities(hq, hkv, s2):
    """Exact per-head identities (any mask): <dQ,Q> = <dK,K>, <dV,V> = <dO,O>, sum_j dK_j = 0."""
    S, D = 32, 8
    q, k, v, do = (_rand((1, S, h, D), s) for h, s in ((hq, 80), (hkv, 81), (hkv, 82), (hq, 83)))
    dq, dk, dv, o, _ = attention_backward(q, k, v, do, s2=s2)
    grp = hq // hkv
    for kh in range(hkv):
        hs = slice(kh * grp, (kh + 1) * grp)
        assert np.sum(dq[:, :, hs] * q[:, :, hs]) == pytest.approx(np.sum(dk[:, :, kh] * k[:, :, kh]), abs=1e-11)
        assert np.sum(dv[:, :, kh] * v[:, :, kh]) == pytest.approx(np.sum(do[:, :, hs] * o[:, :, hs]), abs=1e-11)
        np.testing.assert_allclose(dk[0, :, kh].sum(axis=0), 0.0, atol=1e-12)


# ---------------------------------------------------------------- GQA and S2

def test_gqa_equals_repeated_mha():
    S, D = 40, 8
    q, do = _rand((1, S, 8, D), 90), _rand((1, S, 8, D), 93)
    k, v = _rand((1, S, 2, D), 91), _rand((1, S, 2, D), 92)
    kr, vr = np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2)
    o1, l1 = attention_forward(q, k, v)
    o2, l2 = attention_forward(q, kr, vr)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    dq1, dk1, dv1, _, _ = attention_backward(q, k, v, do)
    dq2, dk2, dv2, _, _ = attention_backward(q, kr, vr, do)
    np.testing.assert_allclose(dq1, dq2, atol=1e-13)
    np.testing.assert_allclose(dk1, dk2.reshape(1, S, 2, 4, D).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(dv1, dv2.reshape(1, S, 2, 4, D).sum(axis=3), atol=1e-13)


def test_s2_full_group_no_shift_is_causal():
    S, H, D = 32, 4, 8
    q, k, v = (_rand((1, S, H, D), s) for s in (100, 101, 102))
    o1, l1 = attention_forward(q, k, v, s2=S2Spec(group=S, shift_head0=H, seqlen=S))
    o2, l2 = attention_forward(q, k, v)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def _sdpa_grouped(q, k, v, G):
    """torch causal SDPA on each group slice separately (float64)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).permute(0, 2, 1, 3)
    outs = []
    for g0 in range(0, q.shape[1], G):
        r = torch.nn.functional.scaled_dot_product_attention(
            t(q[:, g0:g0 + G]), t(k[:, g0:g0 + G]), t(v[:, g0:g0 + G]), is_causal=True)
        outs.append(r.permute(0, 2, 1, 3).numpy())
    return np.concatenate(outs, axis=1)


def test_s2_unshifted_heads_are_grouped_causal():
    S, H, D, G = 48, 4, 8, 12
    q, k, v = (_rand((1, S, H, D), s) for s in (110, 111, 112))
    o, _ = attention_forward(q, k, v, s2=S2Spec(group=G, shift_head0=2, seqlen=S))
    ref = _sdpa_grouped(q[:, :, :2], k[:, :, :2], v[:, :, :2], G)
    np.testing.assert_allclose(o[:, :, :2], ref, atol=1e-12)


def test_s2_shifted_heads_roll_group_rollback():
    """Shifted heads: roll by -G/2, grouped causal attention, roll back (torch.roll + SDPA)."""
    S, H, D, G = 48, 4, 8, 12
    q, k, v = (_rand((1, S, H, D), s) for s in (120, 121, 122))
    o, _ = attention_forward(q, k, v, s2=S2Spec(group=G, shift_head0=2, seqlen=S))
    roll = lambda a, n: np.roll(a, n, axis=1)
    ref = _sdpa_grouped(roll(q[:, :, 2:], -G // 2), roll(k[:, :, 2:], -G // 2), roll(v[:, :, 2:], -G // 2), G)
    np.testing.assert_allclose(o[:, :, 2:], roll(ref, G // 2), atol=1e-12)


def test_s2_shift_direction_immaterial():
    """With G | S, rolling by +G/2 instead of -G/2 only relabels whole groups."""
    S, H, D, G = 48, 2, 8, 12
    q, k, v = (_rand((1, S, H, D), s) for s in (130, 131, 132))
    o, _ = attention_forward(q, k, v, s2=S2Spec(group=G, shift_head0=0, seqlen=S))
    roll = lambda a, n: np.roll(a, n, axis=1)
    ref = _sdpa_grouped(roll(q, G // 2), roll(k, G // 2), roll(v, G // 2), G)
    np.testing.assert_allclose(o, roll(ref, -G // 2), atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant typical mistakes in the oracle (on the CPU) and check that a pin fails."""
    import oracle.attention as oa
    g = _load("handworked_forward.json")
    q = np.array(g["q"]).reshape(1, 3, 1, 1)
    k = np.array(g["k"]).reshape(1, 3, 1, 1)
    v = np.array(g["v"]).reshape(1, 3, 1, 1)
    good = oa.allowed_mask
    # 1) strict causal mask (diagonal excluded)
    monkeypatch.setattr(oa, "allowed_mask", lambda qp, kp, **kw: good(qp, kp, **kw) & (
        np.asarray(kp)[None, :] != np.asarray(qp)[:, None]))
    o, _ = oa.attention_forward(q, k, v, scale=1.0)
    assert not np.allclose(o[0, 1:, 0, 0], g["o"][1:], atol=1e-6)
    monkeypatch.setattr(oa, "allowed_mask", good)
    # 2) dropped Delta term in dS breaks the sum_j dK_j = 0 identity
    S, D = 16, 4
    qq, kk, vv, dd = (_rand((1, S, 1, D), s) for s in (140, 141, 142, 143))
    tau = default_scale(D)
    s = tau * qq[0, :, 0] @ kk[0, :, 0].T
    p, _ = oa._softmax_rows(s, allowed_mask(np.arange(S), np.arange(S)))
    ds_wrong = p * (dd[0, :, 0] @ vv[0, :, 0].T)
    assert np.abs((tau * ds_wrong.T @ qq[0, :, 0]).sum(axis=0)).max() > 1e-3


@pytest.mark.parametrize("mistake", ["reshape_not_transpose", "head_shifted", "row_shifted",
                                     "batch_swapped", "summed_over_rows"])
def test_delta_pin_catches_planted_mistakes(mistake):
    # plausible mistakes in Delta = rowsum(dO * O), each planted in a stand-in for the oracle's
    # backward_delta; the brute-force pin must reject every one
    def bad(o, do):
        prod = o * do
        if mistake == "reshape_not_transpose":     # [B, S, H] reinterpreted as [B, H, S]
            return np.sum(prod, axis=-1).reshape(o.shape[0], o.shape[2], o.shape[1])
        if mistake == "head_shifted":              # dO of the neighbouring head
            return np.transpose(np.sum(o * np.roll(do, 1, axis=2), axis=-1), (0, 2, 1))
        if mistake == "row_shifted":               # dO of the previous row
            return np.transpose(np.sum(o * np.roll(do, 1, axis=1), axis=-1), (0, 2, 1))
        if mistake == "batch_swapped":
            return np.transpose(np.sum(o * do[::-1], axis=-1), (0, 2, 1))
        return np.transpose(np.broadcast_to(np.sum(prod, axis=(1, 3))[:, None, :],
                                            prod.shape[:3]), (0, 2, 1))
    with pytest.raises(AssertionError):
        _check_backward_delta(bad)


# ---------------------------------------------------------------- sampled backward helpers

@pytest.mark.parametrize("hq,hkv,s2", [(2, 2, None), (4, 2, None), (4, 4, S2Spec(8, 2, 32))])
def test_sampled_backward_helpers_match_full(hq, hkv, s2):
    from oracle import backward_delta, cols_backward_dkdv, rows_backward_dq
    S, D = 32, 8
    q, k, v, do = (_rand((1, S, h, D), s) for h, s in ((hq, 150), (hkv, 151), (hkv, 152), (hq, 153)))
    dq, dk, dv, o, _ = attention_backward(q, k, v, do, s2=s2)
    rows = [0, 3, 17, 31]
    for h in range(hq):
        np.testing.assert_allclose(rows_backward_dq(q, k, v, do, 0, h, rows, s2=s2), dq[0, rows, h], atol=1e-13)
    keys = [0, 5, 30, 31]
    for kh in range(hkv):
        dks, dvs = cols_backward_dkdv(q, k, v, do, 0, kh, keys, s2=s2, row_block=7)
        np.testing.assert_allclose(dks, dk[0, keys, kh], atol=1e-13)
        np.testing.assert_allclose(dvs, dv[0, keys, kh], atol=1e-13)
    np.testing.assert_allclose(backward_delta(o, do)[0, 0], np.sum(o[0, :, 0] * do[0, :, 0], axis=-1), atol=1e-14)
