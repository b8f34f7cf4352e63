"""Pins for the oracle's transformer layer (oracle/layer.py): torch autograd in
float64 on the CPU for the dropout-free layer (library routines: layer_norm,
scaled_dot_product_attention, gelu, matmul), and central finite differences
with dropout on (the masks are fixed by the seed, so the layer is smooth)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import layer as ol


def _setup(s=16, b=2, h=32, hq=4, d=8, ffn=64, p_attn=0.0, p_hidden=0.0, causal=True, seed=3):
    rng = np.random.default_rng(seed)
    hd = hq * d
    w = {"gamma1": rng.uniform(0.8, 1.2, h), "beta1": rng.normal(0, 0.1, h),
         "w_qkv": rng.normal(0, 1 / math.sqrt(h), (h, 3 * hd)), "w_o": rng.normal(0, 1 / math.sqrt(hd), (hd, h)),
         "gamma2": rng.uniform(0.8, 1.2, h), "beta2": rng.normal(0, 0.1, h),
         "w_1": rng.normal(0, 1 / math.sqrt(h), (h, ffn)), "w_2": rng.normal(0, 1 / math.sqrt(ffn), (ffn, h)),
         "gamma3": rng.uniform(0.8, 1.2, h), "beta3": rng.normal(0, 0.1, h)}
    cfg = dict(hq=hq, d=d, causal=causal, p_attn=p_attn, p_hidden=p_hidden, seed=11, eps=1e-5)
    x = rng.normal(0, 1, (s, b, h))
    dh2 = rng.normal(0, 1, (s, b, h))
    du3 = rng.normal(0, 1, (s, b, h))
    return x, w, cfg, dh2, du3


def _torch_layer(x, w, cfg):
    s, b, h = x.shape
    hq, d = cfg["hq"], cfg["d"]
    hd = hq * d
    ln = lambda t, gm, bt: F.layer_norm(t, (h,), gm, bt, eps=cfg["eps"])
    u1 = ln(x, w["gamma1"], w["beta1"])
    qkv = u1.reshape(s * b, h) @ w["w_qkv"]
    q, k, v = (qkv[:, i * hd:(i + 1) * hd].reshape(s, b, hq, d).permute(1, 2, 0, 3) for i in range(3))
    o = F.scaled_dot_product_attention(q, k, v, is_causal=cfg["causal"], scale=1.0 / math.sqrt(d))
    a = (o.permute(2, 0, 1, 3).reshape(s * b, hd) @ w["w_o"]).reshape(s, b, h)
    h1 = x + a
    u2 = ln(h1, w["gamma2"], w["beta2"])
    m = (F.gelu(u2.reshape(s * b, h) @ w["w_1"]) @ w["w_2"]).reshape(s, b, h)
    h2 = h1 + m
    return h2, ln(h2, w["gamma3"], w["beta3"])


@pytest.mark.parametrize("causal", [True, False])
def test_dropout_free_layer_equals_torch_autograd(causal):
    x, w, cfg, dh2, du3 = _setup(causal=causal)
    h2, u3, cache = ol.layer_fwd(x, w, cfg)
    dx, g = ol.layer_bwd(dh2, du3, w, cfg, cache)
    tx = torch.tensor(x, requires_grad=True)
    tw = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    th2, tu3 = _torch_layer(tx, tw, cfg)
    np.testing.assert_allclose(h2, th2.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(u3, tu3.detach().numpy(), rtol=0, atol=1e-12)
    ((th2 * torch.tensor(dh2)).sum() + (tu3 * torch.tensor(du3)).sum()).backward()
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=0, atol=1e-10)
    for k in ol.WEIGHTS:
        np.testing.assert_allclose(g[k], tw[k].grad.numpy(), rtol=0, atol=1e-10, err_msg=k)


def test_finite_differences_with_both_dropouts():
    x, w, cfg, dh2, du3 = _setup(s=8, b=1, h=16, hq=2, d=4, ffn=16, p_attn=0.25, p_hidden=0.2)
    h2, u3, cache = ol.layer_fwd(x, w, cfg)
    dx, g = ol.layer_bwd(dh2, du3, w, cfg, cache)

    def loss(xx, ww):
        a, c, _ = ol.layer_fwd(xx, ww, cfg)
        return float((a * dh2).sum() + (c * du3).sum())

    eps = 1e-6
    rng = np.random.default_rng(0)
    for _ in range(6):
        i = tuple(rng.integers(0, n) for n in x.shape)
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        fd = (loss(xp, w) - loss(xm, w)) / (2 * eps)
        assert fd == pytest.approx(dx[i], rel=1e-6, abs=1e-8)
    for k in ("w_qkv", "w_o", "w_1", "w_2", "gamma2", "beta3"):
        i = tuple(rng.integers(0, n) for n in w[k].shape)
        wp = {**w, k: w[k].copy()}
        wm = {**w, k: w[k].copy()}
        wp[k][i] += eps
        wm[k][i] -= eps
        fd = (loss(x, wp) - loss(x, wm)) / (2 * eps)
        assert fd == pytest.approx(g[k][i], rel=1e-6, abs=1e-8), k


def test_dropout_changes_the_layer_and_is_reproducible():
    x, w, cfg, _, _ = _setup(p_attn=0.2, p_hidden=0.2)
    a, _, _ = ol.layer_fwd(x, w, cfg)
    b, _, _ = ol.layer_fwd(x, w, cfg)
    c, _, _ = ol.layer_fwd(x, w, dict(cfg, p_attn=0.0, p_hidden=0.0))
    assert np.array_equal(a, b) and not np.allclose(a, c)
