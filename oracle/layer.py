"""Oracle: one transformer layer around the attention core, float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module.

The layer of the pages' GPT models as one tensor-parallel rank computes it,
without the collectives (LIT-736 record, Key takeaways bullets 1-2: the
layer norms and the dropouts after attention and the MLP form the regions
that sequence parallelism splits; the GEMMs and the attention core sit
between them):

    (x, u1)  = region(resid = x, y = 0)          LN1 (no dropout: p = 0, site 0)
    q, k, v  = split(u1 W_qkv)                   column-parallel GEMM
    o        = attention core (causal, softmax dropout p_attn)
    a        = o W_o                             row-parallel GEMM
    (h1, u2) = region(resid = x,  y = a)         hidden dropout (site 1) + residual + LN2
    z        = u2 W_1 ;  f = GeLU(z)             column-parallel GEMM, exact (erf) GeLU
    m        = f W_2                             row-parallel GEMM
    (h2, u3) = region(resid = h1, y = m)         hidden dropout (site 2) + residual + LN3

The layer returns h2 (the residual stream) and u3 (the next layer's LN1
output).  Weights have no biases (a bias belongs to its GEMM's epilogue).
Activations are [s, b, h]; W_qkv's columns are [q | k | v], each hq * d wide,
head-major.  The region and the attention core are the oracle's own
(oracle.norm, oracle.attention); the backward pass is the chain rule written
out, GEMM by GEMM.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

from . import attention as oat
from . import norm as onm

WEIGHTS = ("gamma1", "beta1", "w_qkv", "w_o", "gamma2", "beta2", "w_1", "w_2", "gamma3", "beta3")


def gelu(z):
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def gelu_grad(z):
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def _region_kw(cfg, site, p):
    return dict(norm="layernorm", p_drop=p, seed=cfg["seed"], site=site)


def layer_fwd(x, w, cfg):
    """x: [s, b, h]; w: dict of WEIGHTS; cfg: hq, d, causal, p_attn, p_hidden, seed, eps.
    Returns (h2, u3, cache)."""
    x = np.asarray(x, dtype=np.float64)
    s, b, h = x.shape
    hq, d = cfg["hq"], cfg["d"]
    hd = hq * d
    eps = cfg["eps"]
    zero = np.zeros_like(x)
    _, u1, m1, r1 = onm.sp_norm_fwd(x, zero, w["gamma1"], w["beta1"], eps=eps, **_region_kw(cfg, 0, 0.0))
    X1 = u1.reshape(s * b, h)
    QKV = X1 @ w["w_qkv"]
    q, k, v = (QKV[:, i * hd:(i + 1) * hd].reshape(s, b, hq, d).transpose(1, 0, 2, 3) for i in range(3))
    akw = dict(causal=cfg["causal"], scale=1.0 / math.sqrt(d), p_drop=cfg["p_attn"], seed=cfg["seed"])
    o, lse = oat.attn_fwd(q, k, v, **akw)
    O2 = o.transpose(1, 0, 2, 3).reshape(s * b, hd)
    A = (O2 @ w["w_o"]).reshape(s, b, h)
    h1, u2, m2, r2 = onm.sp_norm_fwd(x, A, w["gamma2"], w["beta2"], eps=eps, **_region_kw(cfg, 1, cfg["p_hidden"]))
    X2 = u2.reshape(s * b, h)
    Z = X2 @ w["w_1"]
    F = gelu(Z)
    Mo = (F @ w["w_2"]).reshape(s, b, h)
    h2, u3, m3, r3 = onm.sp_norm_fwd(h1, Mo, w["gamma3"], w["beta3"], eps=eps, **_region_kw(cfg, 2, cfg["p_hidden"]))
    cache = dict(x=x, m1=m1, r1=r1, X1=X1, q=q, k=k, v=v, lse=lse, akw=akw, O2=O2, h1=h1, m2=m2, r2=r2,
                 X2=X2, Z=Z, F=F, h2=h2, m3=m3, r3=r3)
    return h2, u3, cache


def layer_bwd(dh2, du3, w, cfg, cache):
    """Gradients of <dh2, h2> + <du3, u3>: returns (dx, dict of weight gradients)."""
    c = cache
    s, b, h = c["x"].shape
    hq, d = cfg["hq"], cfg["d"]
    hd = hq * d
    g = {}
    # LN3 region: grads into h1 (residual) and m (hidden dropout of site 2)
    dh1, dMo, g["gamma3"], g["beta3"] = onm.sp_norm_bwd(du3, dh2, c["h2"], w["gamma3"], c["m3"], c["r3"],
                                                       **_region_kw(cfg, 2, cfg["p_hidden"]))
    dMo = dMo.reshape(s * b, h)
    g["w_2"] = c["F"].T @ dMo
    dZ = (dMo @ w["w_2"].T) * gelu_grad(c["Z"])
    g["w_1"] = c["X2"].T @ dZ
    dX2 = (dZ @ w["w_1"].T).reshape(s, b, h)
    # LN2 region: grads into x (residual) and a
    dx_res, dA, g["gamma2"], g["beta2"] = onm.sp_norm_bwd(dX2, dh1, c["h1"], w["gamma2"], c["m2"], c["r2"],
                                                         **_region_kw(cfg, 1, cfg["p_hidden"]))
    dA = dA.reshape(s * b, h)
    g["w_o"] = c["O2"].T @ dA
    do = (dA @ w["w_o"].T).reshape(s, b, hq, d).transpose(1, 0, 2, 3)
    dq, dk, dv = oat.attn_bwd(c["q"], c["k"], c["v"], c["lse"], do, **c["akw"])
    dQKV = np.concatenate([t.transpose(1, 0, 2, 3).reshape(s * b, hd) for t in (dq, dk, dv)], axis=1)
    g["w_qkv"] = c["X1"].T @ dQKV
    dX1 = (dQKV @ w["w_qkv"].T).reshape(s, b, h)
    # LN1 region (y = 0): its residual output is x itself, unused downstream
    dx, _, g["gamma1"], g["beta1"] = onm.sp_norm_bwd(dX1, dx_res, c["x"], w["gamma1"], c["m1"], c["r1"],
                                                    **_region_kw(cfg, 0, 0.0))
    return dx, g
