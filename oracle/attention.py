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

Padded batches: with ``seqlens`` (one valid length L_b <= s per batch
element) the core acts on the first L_b positions of each element only, as
if the sequence were that long -- keys at or past L_b are invisible, the
dropout mask keeps its global (row, column) counters -- and the padded
positions get O = 0, LSE = -inf and zero gradients.
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


def _lengths(seqlens, b, s):
    if seqlens is None:
        return [s] * b
    L = [int(x) for x in np.asarray(seqlens).reshape(-1)]
    if len(L) != b or any(x < 0 or x > s for x in L):
        raise ValueError("seqlens must hold b lengths in [0, s]")
    return L


def attn_fwd(q, k, v, *, causal, scale, p_drop, seed, head_offset=0, heads=None, seqlens=None):
    """O and LSE.  `heads` optionally restricts the work to [(bb, hh), ...];
    `seqlens` gives each batch element's valid length (padded batch)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    b, s, hq, hkv, d = _check(q, k, v)
    lens = _lengths(seqlens, b, s)
    grp = hq // hkv
    O = np.zeros((b, s, hq, d))
    LSE = np.full((b, hq, s), -np.inf)
    todo = heads if heads is not None else [(bb, hh) for bb in range(b) for hh in range(hq)]
    for bb, hh in todo:
        g, L = hh // grp, lens[bb]
        if L == 0:
            continue
        P, lse = softmax_rows(scores(q[bb, :L, hh], k[bb, :L, g], scale, causal))
        M = attn_keep_mask(seed, p_drop, bb, head_offset + hh, L, L)
        Pd = P * M / (1.0 - p_drop)
        O[bb, :L, hh] = Pd @ v[bb, :L, g]
        LSE[bb, hh, :L] = lse
    return O, LSE


def attn_probs(q, k, *, causal, scale, bb, hh, hkv_index=None):
    """P (undropped softmax) for one (batch, q-head); used by the pins."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    g = hh // (q.shape[2] // k.shape[2]) if hkv_index is None else hkv_index
    return softmax_rows(scores(q[bb, :, hh], k[bb, :, g], scale, causal))


def attn_bwd(q, k, v, lse, do, *, causal, scale, p_drop, seed, head_offset=0,
             heads=None, seqlens=None):
    """dQ, dK, dV by recomputation: P = exp(S - LSE), M regenerated from Philox.

    This is the selective-recompute backward: neither P nor M is an input.
    `lse` is the forward's LSE (``[b, hq, s]``); `seqlens` as in attn_fwd.
    """
    q, k, v, do, lse = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do, lse))
    b, s, hq, hkv, d = _check(q, k, v)
    lens = _lengths(seqlens, b, s)
    grp = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    todo = heads if heads is not None else [(bb, hh) for bb in range(b) for hh in range(hq)]
    for bb, hh in todo:
        g, L = hh // grp, lens[bb]
        if L == 0:
            continue
        S = scores(q[bb, :L, hh], k[bb, :L, g], scale, causal)
        P = np.exp(S - lse[bb, hh, :L][:, None])
        M = attn_keep_mask(seed, p_drop, bb, head_offset + hh, L, L)
        dq[bb, :L, hh], dk_h, dv_h = _bwd_from_probs(P, M, p_drop, q[bb, :L, hh], k[bb, :L, g],
                                                     v[bb, :L, g], do[bb, :L, hh], scale)
        dk[bb, :L, g] += dk_h
        dv[bb, :L, g] += dv_h
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
