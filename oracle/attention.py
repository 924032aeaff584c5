"""Plain float64 softmax attention: the oracle the HIP path is checked against.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Nothing here is blocked,
fused or reordered beyond the definition: every query row materialises its
whole row of scores over the allowed keys, takes one max, one sum and one
division.  Rows are processed in groups purely to bound memory.

What is computed, and where it comes from
-----------------------------------------
* Exact softmax attention.  The Ring Attention page (research.elamur.ai summary
  of "Ring Attention with Blockwise Transformers for Near-Infinite Context",
  section Summary) states that blockwise attention stays exact and gives the
  same result whatever order the key/value blocks are processed in; the
  long-context recipe page (sourcepulse.org project page, section "How It
  Works") stresses full attention with no approximation.  The blockwise method
  therefore reaches the plain definition, which is what this module evaluates.
* Partial (output, log-sum-exp) pairs and their merge: the order independence
  in the same Summary is realised by carrying, per query row, the pair
  (O_i, LSE_i) of a block of keys and combining two pairs with log-add-exp
  weights.
* S2-Attn: the LongLoRA page (research.elamur.ai summary of "LongLoRA:
  Efficient Fine-tuning of Long-Context Large Language Models", section
  Summary) splits tokens into groups, attends inside each group, and in half
  of the heads shifts tokens by half a group; section "Key points" gives group
  2048 for 8192-token training.
* Backward: the pages train with this attention (full fine-tuning on the
  project page, S2 fine-tuning on the LongLoRA page, a 512K fine-tune on the
  Ring Attention page) but print no gradient formula.  The gradient of the
  scalar <dO, O> with respect to Q, K and V is used (LSE is not
  differentiated).

Readings taken where the pages are silent
-----------------------------------------
1. Softmax scale tau = 1/sqrt(D) unless given.
2. Causal: 0-based global positions, key j allowed for query i iff pos(j) <= pos(i).
3. LSE is the natural log of the sum of exp of the scaled scores, shape [B, Hq, S].
4. A row with no allowed key in a partial has (O, LSE) = (0, -inf); the merge
   treats that pair as the identity.
5. GQA: query head h reads key/value head h // (Hq / Hkv).
6. S2: shifted heads are [shift_head0, Hq); rolled position rho(p) = (p - G/2) mod S;
   keys allowed iff same group of rolled positions and rho(j) <= rho(i).  Results
   are indexed by original positions.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

NEG_INF = -np.inf


def default_scale(head_dim: int) -> float:
    """Softmax temperature 1/sqrt(D) (reading 1)."""
    return 1.0 / math.sqrt(head_dim)


@dataclass(frozen=True)
class S2Spec:
    """Shifted sparse attention layout (LongLoRA page, Summary and Key points).

    group: tokens per group G (must divide seqlen, must be even)
    shift_head0: heads [shift_head0, Hq) are shifted by G/2
    seqlen: total sequence length S the roll wraps around
    """
    group: int
    shift_head0: int
    seqlen: int

    def shift_for_head(self, head: int) -> int:
        return self.group // 2 if head >= self.shift_head0 else 0


def allowed_mask(q_pos: np.ndarray, k_pos: np.ndarray, *, causal: bool = True,
                 s2: Optional[S2Spec] = None, head: int = 0) -> np.ndarray:
    """Boolean [len(q_pos), len(k_pos)]: which (query, key) pairs attend (readings 2, 6)."""
    qp = np.asarray(q_pos, dtype=np.int64)[:, None]
    kp = np.asarray(k_pos, dtype=np.int64)[None, :]
    if s2 is not None:
        shift = s2.shift_for_head(head)
        rq = (qp - shift) % s2.seqlen
        rk = (kp - shift) % s2.seqlen
        return (rq // s2.group == rk // s2.group) & (rk <= rq)
    if causal:
        return kp <= qp
    return np.ones((qp.shape[0], kp.shape[1]), dtype=bool)


def _softmax_rows(scores: np.ndarray, mask: np.ndarray):
    """Probabilities and LSE of each row of masked scores; empty rows -> (0, -inf)."""
    s = np.where(mask, scores, NEG_INF)
    m = s.max(axis=1)
    nonempty = np.isfinite(m)
    m_safe = np.where(nonempty, m, 0.0)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for masked pairs
    z = e.sum(axis=1)
    z_safe = np.where(nonempty, z, 1.0)
    lse = np.where(nonempty, m_safe + np.log(z_safe), NEG_INF)
    p = e / z_safe[:, None]
    return p, lse


def _kv_head(h: int, hq: int, hkv: int) -> int:
    if hq % hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    return h // (hq // hkv)


def rows_forward(q, k, v, b: int, h: int, rows: Sequence[int], *, scale=None, causal=True,
                 q_pos0: int = 0, k_pos0: int = 0, s2: Optional[S2Spec] = None):
    """O [len(rows), D] and LSE [len(rows)] of selected query rows of one (batch, head).

    Used to check single outputs of runs too large for the whole oracle.
    """
    _, _, hq, d = q.shape
    hkv = k.shape[2]
    tau = default_scale(d) if scale is None else float(scale)
    kvh = _kv_head(h, hq, hkv)
    rows = np.asarray(rows, dtype=np.int64)
    # slice first, then upcast: only the rows and the one key/value head are needed
    Q = np.asarray(q[b, rows, h, :], dtype=np.float64)
    K = np.asarray(k[b, :, kvh, :], dtype=np.float64)
    V = np.asarray(v[b, :, kvh, :], dtype=np.float64)
    k_pos = k_pos0 + np.arange(K.shape[0])
    s = tau * (Q @ K.T)
    p, lse = _softmax_rows(s, allowed_mask(q_pos0 + rows, k_pos, causal=causal, s2=s2, head=h))
    return p @ V, lse


def attention_forward(q, k, v, *, scale=None, causal: bool = True, q_pos0: int = 0,
                      k_pos0: int = 0, s2: Optional[S2Spec] = None,
                      heads: Optional[Sequence[int]] = None, row_block: int = 512):
    """Exact softmax attention of Q [B,Sq,Hq,D] against K, V [B,Sk,Hkv,D].

    Returns O [B, Sq, len(heads), D] and LSE [B, len(heads), Sq] in float64
    (heads defaults to all query heads).  q_pos0 / k_pos0 are the global
    positions of row 0 of Q and of K/V, so a call on one key/value chunk gives
    that chunk's partial pair (reading 4 for rows the chunk cannot reach).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    heads = list(range(hq)) if heads is None else list(heads)
    tau = default_scale(d) if scale is None else float(scale)
    o = np.zeros((bsz, sq, len(heads), d))
    lse = np.full((bsz, len(heads), sq), NEG_INF)
    k_pos = k_pos0 + np.arange(sk)
    for b in range(bsz):
        for hi, h in enumerate(heads):
            kvh = _kv_head(h, hq, hkv)
            K = k[b, :, kvh, :]
            V = v[b, :, kvh, :]
            for r0 in range(0, sq, row_block):
                r1 = min(sq, r0 + row_block)
                s = tau * (q[b, r0:r1, h, :] @ K.T)
                mask = allowed_mask(q_pos0 + np.arange(r0, r1), k_pos, causal=causal, s2=s2, head=h)
                p, l = _softmax_rows(s, mask)
                o[b, r0:r1, hi, :] = p @ V
                lse[b, hi, r0:r1] = l
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial pairs over disjoint key sets (reading 4).

    L = log(e^La + e^Lb); O = e^(La-L) O_a + e^(Lb-L) O_b.  A pair with LSE = -inf
    contributes nothing, whatever its O holds; two such pairs give (0, -inf).
    o_* are [B, S, H, D], lse_* are [B, H, S].
    """
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    L = np.logaddexp(lse_a, lse_b)
    fin = np.isfinite(L)
    L_safe = np.where(fin, L, 0.0)
    wa = np.where(np.isfinite(lse_a) & fin, np.exp(np.where(np.isfinite(lse_a), lse_a, 0.0) - L_safe), 0.0)
    wb = np.where(np.isfinite(lse_b) & fin, np.exp(np.where(np.isfinite(lse_b), lse_b, 0.0) - L_safe), 0.0)
    # weights are [B, H, S]; outputs are [B, S, H, D]
    wa_t = np.transpose(wa, (0, 2, 1))[..., None]
    wb_t = np.transpose(wb, (0, 2, 1))[..., None]
    oa = np.where(wa_t > 0, np.asarray(o_a, dtype=np.float64), 0.0)
    ob = np.where(wb_t > 0, np.asarray(o_b, dtype=np.float64), 0.0)
    return wa_t * oa + wb_t * ob, np.where(fin, L, NEG_INF)


def ring_attention_forward(q, k, v, order: Sequence[int], chunk_len: int, *, scale=None,
                           causal: bool = True, s2: Optional[S2Spec] = None,
                           heads: Optional[Sequence[int]] = None):
    """The resident query block against key/value chunks visited in `order`.

    Each step computes one chunk's partial pair and merges it into the running
    pair, as the Ring Attention page's Summary describes for one host.
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    bsz, sq, hq, d = q.shape
    nh = hq if heads is None else len(heads)
    o = np.zeros((bsz, sq, nh, d))
    lse = np.full((bsz, nh, sq), NEG_INF)
    sk = k.shape[1]
    for c in order:
        c0, c1 = c * chunk_len, min(sk, (c + 1) * chunk_len)
        oc, lc = attention_forward(q, k[:, c0:c1], v[:, c0:c1], scale=scale, causal=causal,
                                   k_pos0=c0, s2=s2, heads=heads)
        o, lse = lse_merge(o, lse, oc, lc)
    return o, lse


def attention_backward(q, k, v, do, *, scale=None, causal: bool = True,
                       s2: Optional[S2Spec] = None, row_block: int = 512):
    """Gradients of <dO, O> with respect to Q, K, V (analytic; see module docstring).

    With P the attention probabilities and O = P V:
      Delta_i = sum_d dO_id O_id
      dP_ij = dO_i . V_j,   dS_ij = P_ij (dP_ij - Delta_i)
      dQ_i = tau sum_j dS_ij K_j,  dK_j = tau sum_i dS_ij Q_i,  dV_j = sum_i P_ij dO_i
    For GQA, dK and dV of a key/value head sum over the query heads that read it.
    Returns dq [B,Sq,Hq,D], dk, dv [B,Sk,Hkv,D], and the forward (o, lse).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    bsz, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    tau = default_scale(d) if scale is None else float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros_like(q)
    lse = np.full((bsz, hq, sq), NEG_INF)
    k_pos = np.arange(sk)
    for b in range(bsz):
        for h in range(hq):
            kvh = _kv_head(h, hq, hkv)
            K = k[b, :, kvh, :]
            V = v[b, :, kvh, :]
            for r0 in range(0, sq, row_block):
                r1 = min(sq, r0 + row_block)
                Q = q[b, r0:r1, h, :]
                dO = do[b, r0:r1, h, :]
                s = tau * (Q @ K.T)
                mask = allowed_mask(np.arange(r0, r1), k_pos, causal=causal, s2=s2, head=h)
                p, l = _softmax_rows(s, mask)
                O = p @ V
                o[b, r0:r1, h, :] = O
                lse[b, h, r0:r1] = l
                delta = np.sum(dO * O, axis=1)
                dp = dO @ V.T
                ds = p * (dp - delta[:, None])
                dq[b, r0:r1, h, :] = tau * (ds @ K)
                dk[b, :, kvh, :] += tau * (ds.T @ Q)
                dv[b, :, kvh, :] += p.T @ dO
    return dq, dk, dv, o, lse


def backward_delta(o, do):
    """Delta_i = sum_d dO_id O_id, [B, H, S] from [B, S, H, D] inputs (first step of the backward)."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    return np.transpose(np.sum(o * do, axis=-1), (0, 2, 1))


def rows_backward_dq(q, k, v, do, b: int, h: int, rows: Sequence[int], *, scale=None,
                     causal: bool = True, s2: Optional[S2Spec] = None):
    """dQ of selected query rows of one (batch, head), from the definitions above.

    Each row needs only its own full row of probabilities (its LSE), its own
    output O_i (for Delta_i) and every key/value row.
    """
    _, _, hq, d = q.shape
    hkv = k.shape[2]
    tau = default_scale(d) if scale is None else float(scale)
    kvh = _kv_head(h, hq, hkv)
    rows = np.asarray(rows, dtype=np.int64)
    Q = np.asarray(q[b, rows, h, :], dtype=np.float64)
    dO = np.asarray(do[b, rows, h, :], dtype=np.float64)
    K = np.asarray(k[b, :, kvh, :], dtype=np.float64)
    V = np.asarray(v[b, :, kvh, :], dtype=np.float64)
    s = tau * (Q @ K.T)
    p, _ = _softmax_rows(s, allowed_mask(rows, np.arange(K.shape[0]), causal=causal, s2=s2, head=h))
    O = p @ V
    delta = np.sum(dO * O, axis=1)
    ds = p * (dO @ V.T - delta[:, None])
    return tau * (ds @ K)


def cols_backward_dkdv(q, k, v, do, b: int, kvh: int, keys: Sequence[int], *, scale=None,
                       causal: bool = True, s2: Optional[S2Spec] = None, row_block: int = 1024):
    """dK and dV of selected key rows of one (batch, key/value head).

    Needs every query row's LSE and output (all keys), so it runs the plain
    forward over all rows of the query heads that read this key/value head,
    then sums the selected key columns of dS and P over those rows.
    """
    _, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    tau = default_scale(d) if scale is None else float(scale)
    grp = hq // hkv
    keys = np.asarray(keys, dtype=np.int64)
    K = np.asarray(k[b, :, kvh, :], dtype=np.float64)
    V = np.asarray(v[b, :, kvh, :], dtype=np.float64)
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    for h in range(kvh * grp, (kvh + 1) * grp):
        for r0 in range(0, sq, row_block):
            r1 = min(sq, r0 + row_block)
            Q = np.asarray(q[b, r0:r1, h, :], dtype=np.float64)
            dO = np.asarray(do[b, r0:r1, h, :], dtype=np.float64)
            s = tau * (Q @ K.T)
            p, _ = _softmax_rows(s, allowed_mask(np.arange(r0, r1), np.arange(sk), causal=causal, s2=s2, head=h))
            delta = np.sum(dO * (p @ V), axis=1)
            pc = p[:, keys]
            dsc = pc * (dO @ V[keys].T - delta[:, None])
            dk += tau * (dsc.T @ Q)
            dv += pc.T @ dO
    return dk, dv
