"""Oracle: the attention core, forward and backward, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module.

What is computed.  The attention core of a transformer layer -- QK^T, the
softmax, the softmax dropout and the product with V -- is the part that
selective activation recomputation does not store but re-runs in the backward
pass ("Reducing Activation Recomputation in Large Transformer Models", LIT-736
record, Key takeaways bullet 4; "Recomputing Activations" plate, second
paragraph).  Tiling it (FlashAttention, described on the METP page,
Introduction, third paragraph) reorders the same sums exactly, so the oracle is
the plain definition with the full s x s score matrix materialised per
(batch, head):

    S   = Q K^T * scale          (scale = 1/sqrt(d_h); causal: S_ij = -inf, j > i)
    P   = softmax_rows(S),       LSE_i = log sum_j exp(S_ij)   (natural log)
    P_d = P * M / (1 - p)        M = Philox keep-mask (oracle.philox)
    O   = P_d V

Backward, from the chain rule, for upstream gradient dO:

    dV  = P_d^T dO
    dP_d = dO V^T ;  dP = dP_d * M / (1 - p)
    dS  = P * (dP - rowsum(dP * P))
    dQ  = dS K * scale ;  dK = dS^T Q * scale

Grouped-query attention: q-head hh reads kv-head hh // (hq / hkv); dK and dV
of a kv-head sum the contributions of its q-heads.

Layouts: Q, O, dO, dQ ``[b, s, hq, d]``; K, V, dK, dV ``[b, s, hkv, d]``;
LSE ``[b, hq, s]``.  All arithmetic in float64.
"""
from __future__ import annotations

import numpy as np

from .philox import attn_keep_mask


def _check(q, k, v):
    b, s, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[1] != s or k.shape[3] != d:
        raise ValueError("q/k/v shapes disagree")
    hkv = k.shape[2]
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    return b, s, hq, hkv, d


def scores(q_bh, k_bh, scale, causal):
    """S = Q K^T * scale for one (batch, head), with the causal -inf mask."""
    S = (q_bh @ k_bh.T) * scale
    if causal:
        n = S.shape[0]
        S = np.where(np.tril(np.ones((n, n), dtype=bool)), S, -np.inf)
    return S


def softmax_rows(S):
    """Row softmax and its natural-log normaliser LSE."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return E / l, (m + np.log(l))[:, 0]


def attn_fwd(q, k, v, *, causal, scale, p_drop, seed, head_offset=0, heads=None):
    """O and LSE.  `heads` optionally restricts the work to [(bb, hh), ...]."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    b, s, hq, hkv, d = _check(q, k, v)
    grp = hq // hkv
    O = np.zeros((b, s, hq, d))
    LSE = np.zeros((b, hq, s))
    todo = heads if heads is not None else [(bb, hh) for bb in range(b) for hh in range(hq)]
    for bb, hh in todo:
        g = hh // grp
        P, lse = softmax_rows(scores(q[bb, :, hh], k[bb, :, g], scale, causal))
        M = attn_keep_mask(seed, p_drop, bb, head_offset + hh, s, s)
        Pd = P * M / (1.0 - p_drop)
        O[bb, :, hh] = Pd @ v[bb, :, g]
        LSE[bb, hh] = lse
    return O, LSE


def attn_probs(q, k, *, causal, scale, bb, hh, hkv_index=None):
    """P (undropped softmax) for one (batch, q-head); used by the pins."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    g = hh // (q.shape[2] // k.shape[2]) if hkv_index is None else hkv_index
    return softmax_rows(scores(q[bb, :, hh], k[bb, :, g], scale, causal))


def attn_bwd(q, k, v, lse, do, *, causal, scale, p_drop, seed, head_offset=0,
             heads=None):
    """dQ, dK, dV by recomputation: P = exp(S - LSE), M regenerated from Philox.

    This is the selective-recompute backward: neither P nor M is an input.
    `lse` is the forward's LSE (``[b, hq, s]``).
    """
    q, k, v, do, lse = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do, lse))
    b, s, hq, hkv, d = _check(q, k, v)
    grp = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    todo = heads if heads is not None else [(bb, hh) for bb in range(b) for hh in range(hq)]
    for bb, hh in todo:
        g = hh // grp
        S = scores(q[bb, :, hh], k[bb, :, g], scale, causal)
        P = np.exp(S - lse[bb, hh][:, None])
        M = attn_keep_mask(seed, p_drop, bb, head_offset + hh, s, s)
        dq[bb, :, hh], dk_h, dv_h = _bwd_from_probs(P, M, p_drop, q[bb, :, hh], k[bb, :, g],
                                                    v[bb, :, g], do[bb, :, hh], scale)
        dk[bb, :, g] += dk_h
        dv[bb, :, g] += dv_h
    return dq, dk, dv


def _bwd_from_probs(P, M, p_drop, q_bh, k_bh, v_bh, do_bh, scale):
    keep_scale = M / (1.0 - p_drop)
    Pd = P * keep_scale
    dv = Pd.T @ do_bh
    dP = (do_bh @ v_bh.T) * keep_scale
    dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
    dq = (dS @ k_bh) * scale
    dk = (dS.T @ q_bh) * scale
    return dq, dk, dv


def attn_bwd_stored(P, M, q_bh, k_bh, v_bh, do_bh, *, scale, p_drop):
    """The same backward for one (batch, head) from a STORED P and mask.

    This is what no recomputation would keep (the 5as^2b bytes); the pins
    check that the recompute path above gives the same gradients.
    """
    return _bwd_from_probs(np.asarray(P, np.float64), np.asarray(M), p_drop,
                           *(np.asarray(x, np.float64) for x in (q_bh, k_bh, v_bh, do_bh)),
                           scale)
