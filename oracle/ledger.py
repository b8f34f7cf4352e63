"""Oracle: the activation-memory ledger of one transformer layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module.

Bytes of stored activations per layer for sequence length s, micro-batch b,
hidden size h, a attention heads and tensor-parallel size t (2-byte
activations):

* no recomputation:          sbh (34 + 5 a s / h)   -- the plate's per-token
  byte formula ("Recomputing Activations" plate, "What you will learn")
  multiplied by s b
* selective recomputation:   34 sbh                  (attention scores re-done)
* full recomputation:        2 sbh                   (each layer's input only)
* tensor parallel only:      sbh (10 + 24/t + 5 a s / (h t)); the layer norms and
  the post-attention / post-MLP dropouts, 10sbh, are replicated on every rank
  (LIT-736 record, Key takeaways bullet 1)
* tensor + sequence parallel: the unparallelised figure divided by t
  (LIT-736 record, Key takeaways bullet 2)

The split of 34 into 10 replicated + 24 divided by t, and of the attention
term into three a*s^2*b tensors (softmax output 2, dropout mask 1, dropout
output 2 bytes per element), are the reading that makes the pages' totals
consistent; the pages print only the totals.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

REPLICATED_PER_SBH = 10        # LN inputs (4) + post-attn/MLP dropout masks (2) + QKV/fc1 inputs (4)
SPLIT_PER_SBH = 24             # the rest of the 34
ATTN_SCORE_PER_AS2B = 5        # softmax out (2) + dropout mask (1) + dropout out (2)


@dataclass(frozen=True)
class LayerDims:
    s: int
    b: int
    h: int
    a: int


def bytes_none(d: LayerDims) -> float:
    return d.s * d.b * d.h * (34 + 5 * d.a * d.s / d.h)


def bytes_selective(d: LayerDims) -> float:
    return 34.0 * d.s * d.b * d.h


def bytes_full(d: LayerDims) -> float:
    return 2.0 * d.s * d.b * d.h


def bytes_tp(d: LayerDims, t: int, selective: bool = False) -> float:
    """Tensor parallel without sequence parallel: the 10sbh term stays whole."""
    sbh = d.s * d.b * d.h
    attn = 0.0 if selective else ATTN_SCORE_PER_AS2B * d.a * d.s * d.s * d.b / t
    return REPLICATED_PER_SBH * sbh + SPLIT_PER_SBH * sbh / t + attn


def bytes_tp_sp(d: LayerDims, t: int, selective: bool = False) -> float:
    """Tensor + sequence parallel: every term divides by t."""
    return (bytes_selective(d) if selective else bytes_none(d)) / t


def per_token_bytes(d_model: int, heads: int, seq: int, mode: str) -> float:
    """The per-token, per-layer form: 34 d + 5 H T / 34 d / 2 d."""
    if mode == "none":
        return 34 * d_model + 5 * heads * seq
    if mode == "selective":
        return 34 * d_model
    if mode == "full":
        return 2 * d_model
    raise ValueError(mode)


def model_bytes(d: LayerDims, layers: int, mode: str) -> float:
    f = {"none": bytes_none, "selective": bytes_selective, "full": bytes_full}[mode]
    return layers * f(d)


def full_recompute_flops_ratio() -> float:
    """A second forward pass on top of forward + backward (2N + 4N per token)
    adds 2N, a third of the training FLOPs."""
    return 8.0 / 6.0


def selective_recompute_extra(n_params: float, d: LayerDims, layers: int,
                              causal: bool = True) -> float:
    """Extra compute of re-doing the score FLOPs (QK^T and PV forward).

    Reading of the plate's "selective figure is the attention-score FLOPs
    re-done": forward score FLOPs per token per layer are 4 s h (2 s h causal);
    the base is 6N plus the attention FLOPs of forward + backward (3x forward).
    """
    fwd = (2.0 if causal else 4.0) * d.s * d.h * layers
    return fwd / (6.0 * n_params + 3.0 * fwd)


def kept_bytes_this_library(s, b, hq, hkv, d_head, *, norm_rows, hidden, dtype_bytes=2,
                            norm="layernorm"):
    """Bytes this library keeps between its forward and backward calls.

    Attention core of one rank (b sequences of s positions): Q and O at hq
    heads, K and V at hkv heads (grouped-query attention shares each kv-head
    among hq / hkv q-heads), all of d_head values in the activation dtype, plus
    the fp32 logsumexp of every (sequence, q-head, position).
    Norm region (norm_rows rows of `hidden` values): h = resid + dropout(y) in
    the activation dtype, plus fp32 mean and rstd per row (rstd only for
    RMSNorm).  No dropout mask is kept (both are regenerated) and no term
    grows with s^2.
    """
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    q_and_o = 2 * b * s * hq * d_head * dtype_bytes
    k_and_v = 2 * b * s * hkv * d_head * dtype_bytes
    lse = 4 * b * hq * s
    h_kept = norm_rows * hidden * dtype_bytes
    stats = (8 if norm == "layernorm" else 4) * norm_rows
    return q_and_o + k_and_v + lse + h_kept + stats


# ---- recompute policy: a per-layer choice of none / selective / full ----------
# The plate's closing paragraphs: in practice the choice between selective
# and full recomputation is left to the user, full recomputation being for
# when memory binds.  The plan below is the plain definition of that choice
# made per layer: of all assignments of the three policies to the layers, the
# one with the least extra compute whose stored bytes fit the budget (ties:
# fewer stored bytes, then fewer fully recomputed layers).  Exact rational
# arithmetic, brute force over counts.

POLICIES = ("none", "selective", "full")


def layer_bytes_exact(s, b, h, a, t, sequence_parallel, policy) -> Fraction:
    """Bytes one layer stores on one of t tensor-parallel ranks.

    none / selective follow bytes_tp / bytes_tp_sp above; full keeps the layer
    input, 2sbh, whole under tensor parallelism alone and its s/t slice with
    sequence parallelism (reading: the input sits in the sequence-parallel
    region)."""
    sbh = Fraction(s * b * h)
    if policy == "full":
        return 2 * sbh / t if sequence_parallel else 2 * sbh
    attn = Fraction(ATTN_SCORE_PER_AS2B * a * s * s * b) if policy == "none" else Fraction(0)
    if sequence_parallel:
        return (34 * sbh + attn) / t
    return REPLICATED_PER_SBH * sbh + (SPLIT_PER_SBH * sbh + attn) / t


def extra_compute_exact(s, h, layers, n_params, causal, n_selective, n_full) -> Fraction:
    """Extra FLOPs over the training FLOPs when n_selective layers re-do their
    attention-score FLOPs (A = 4sh per token, 2sh causal) and n_full layers
    re-do their whole forward pass (2N/L + A: 6N -> 8N per token when all do).
    Base: 6N + 3LA (the base of selective_recompute_extra above)."""
    A = Fraction((2 if causal else 4) * s * h)
    per_full = Fraction(2 * n_params, layers) + A
    return (n_selective * A + n_full * per_full) / (6 * n_params + 3 * layers * A)


def plan_recompute(budget, *, s, b, h, a, layers, n_params=0, t=1, sequence_parallel=False,
                   causal=True):
    """Returns (n_none, n_selective, n_full, bytes, extra) or None if nothing fits."""
    budget = Fraction(budget)
    mem = {p: layer_bytes_exact(s, b, h, a, t, sequence_parallel, p) for p in POLICIES}
    best = None
    for n_full in range(layers + 1):
        for n_sel in range(layers - n_full + 1):
            n_none = layers - n_full - n_sel
            m = n_none * mem["none"] + n_sel * mem["selective"] + n_full * mem["full"]
            if m > budget:
                continue
            x = extra_compute_exact(s, h, layers, n_params, causal, n_sel, n_full)
            key = (x, m, n_full)
            if best is None or key < best[0]:
                best = (key, (n_none, n_sel, n_full, m, x))
    return None if best is None else best[1]
