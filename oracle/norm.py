"""Oracle: the sequence-parallel norm region, forward and backward, float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module.

What is computed.  Under tensor parallelism the layer norms and the dropouts
after attention and after the MLP are not split, so every rank holds them whole
(the 10sbh term); sequence parallelism splits exactly these regions along the
sequence, because they act on each position independently ("Reducing
Activation Recomputation in Large Transformer Models", LIT-736 record, Key
takeaways bullets 1 and 2).  One rank owns rows ``[s_local, b, h]`` of the
sequence, starting at global position ``seq_offset``.

Per row (the region between the attention/MLP output and the next GEMM):

    h = resid + y * M / (1 - p)                (hidden dropout + residual)
    LayerNorm: mu = mean(h), var = mean((h - mu)^2), rstd = 1/sqrt(var + eps)
               u = (h - mu) * rstd * gamma + beta
    RMSNorm:   rstd = 1/sqrt(mean(h^2) + eps),  u = h * rstd * gamma

Backward, for upstream du (into u) and dres (into h from the residual path):

    xhat = (h - mu) * rstd   (RMSNorm: h * rstd);   g = du * gamma
    LayerNorm: dh = rstd * (g - mean(g) - xhat * mean(g * xhat)) + dres
    RMSNorm:   dh = rstd * (g - xhat * mean(g * xhat)) + dres
    dresid = dh ;  dy = dh * M / (1 - p)
    dgamma = sum_rows du * xhat ;  dbeta = sum_rows du

M is the hidden-dropout keep mask of oracle.philox (keyed by global sequence
position, so the split along s does not change it).
"""
from __future__ import annotations

import numpy as np

from .philox import hidden_keep_mask


def sp_norm_fwd(resid, y, gamma, beta, *, norm, eps, p_drop, seed, site, seq_offset=0):
    """h, u ([s_local, b, h]), mean and rstd ([s_local, b]); mean is None for RMSNorm."""
    resid = np.asarray(resid, np.float64)
    y = np.asarray(y, np.float64)
    gamma = np.asarray(gamma, np.float64)
    s_local, b, hdim = resid.shape
    M = hidden_keep_mask(seed, p_drop, site, s_local, b, hdim, seq_offset)
    h = resid + y * M / (1.0 - p_drop)
    if norm == "layernorm":
        mu = h.mean(axis=-1)
        var = ((h - mu[..., None]) ** 2).mean(axis=-1)
        rstd = 1.0 / np.sqrt(var + eps)
        u = (h - mu[..., None]) * rstd[..., None] * gamma + np.asarray(beta, np.float64)
        return h, u, mu, rstd
    if norm == "rmsnorm":
        rstd = 1.0 / np.sqrt((h * h).mean(axis=-1) + eps)
        u = h * rstd[..., None] * gamma
        return h, u, None, rstd
    raise ValueError(norm)


def sp_norm_bwd(du, dres, h, gamma, mean, rstd, *, norm, p_drop, seed, site, seq_offset=0):
    """dresid (= dh), dy, dgamma, dbeta (dbeta is None for RMSNorm)."""
    du = np.asarray(du, np.float64)
    dres = np.asarray(dres, np.float64)
    h = np.asarray(h, np.float64)
    gamma = np.asarray(gamma, np.float64)
    rstd = np.asarray(rstd, np.float64)[..., None]
    s_local, b, hdim = h.shape
    g = du * gamma
    if norm == "layernorm":
        xhat = (h - np.asarray(mean, np.float64)[..., None]) * rstd
        dh = rstd * (g - g.mean(axis=-1, keepdims=True)
                     - xhat * (g * xhat).mean(axis=-1, keepdims=True)) + dres
        dbeta = du.sum(axis=(0, 1))
    elif norm == "rmsnorm":
        xhat = h * rstd
        dh = rstd * (g - xhat * (g * xhat).mean(axis=-1, keepdims=True)) + dres
        dbeta = None
    else:
        raise ValueError(norm)
    M = hidden_keep_mask(seed, p_drop, site, s_local, b, hdim, seq_offset)
    dy = dh * M / (1.0 - p_drop)
    dgamma = (du * xhat).sum(axis=(0, 1))
    return dh, dy, dgamma, dbeta
