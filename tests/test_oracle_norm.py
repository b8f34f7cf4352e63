"""Pins for the oracle's sequence-parallel norm region.

Fixed to torch's F.layer_norm / F.rms_norm and autograd (library routines,
CPU float64), to closed-form invariants of the normalisation backward, to
central finite differences, and to the rocRAND-pinned hidden mask.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import norm as nm
from oracle import philox as ph


def _inputs(s_local, b, h, seed=0):
    rng = np.random.default_rng(seed)
    resid = rng.standard_normal((s_local, b, h))
    y = rng.standard_normal((s_local, b, h))
    du = rng.standard_normal((s_local, b, h))
    dres = rng.standard_normal((s_local, b, h))
    gamma = rng.uniform(0.9, 1.1, h)
    beta = rng.standard_normal(h) * 0.02
    return resid, y, du, dres, gamma, beta


@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_p0_forward_and_backward_equal_torch(norm):
    resid, y, du, dres, gamma, beta = _inputs(6, 3, 40, seed=1)
    kw = dict(norm=norm, p_drop=0.0, seed=0, site=1)
    h, u, mu, rstd = nm.sp_norm_fwd(resid, y, gamma, beta, eps=1e-5, **kw)
    tr = torch.tensor(resid, requires_grad=True)
    ty = torch.tensor(y, requires_grad=True)
    tg = torch.tensor(gamma, requires_grad=True)
    tb = torch.tensor(beta, requires_grad=True)
    th = tr + ty
    if norm == "layernorm":
        tu = F.layer_norm(th, (40,), tg, tb, eps=1e-5)
    else:
        tu = F.rms_norm(th, (40,), tg, eps=1e-5)
    np.testing.assert_allclose(h, th.detach().numpy(), rtol=1e-15)
    np.testing.assert_allclose(u, tu.detach().numpy(), rtol=1e-12, atol=1e-12)
    torch.autograd.backward([tu, th], [torch.tensor(du), torch.tensor(dres)])
    dh, dy, dgamma, dbeta = nm.sp_norm_bwd(du, dres, h, gamma, mu, rstd, **{k: v for k, v in kw.items()})
    np.testing.assert_allclose(dh, tr.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dy, ty.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dgamma, tg.grad.numpy(), rtol=1e-11, atol=1e-12)
    if norm == "layernorm":
        np.testing.assert_allclose(dbeta, tb.grad.numpy(), rtol=1e-11, atol=1e-12)
    else:
        assert dbeta is None


def test_dropout_is_visible_in_h():
    """resid = 0, y = 1 gives h = M / (1 - p) with M the rocRAND-pinned mask."""
    s_local, b, hd, p = 8, 2, 48, 0.25
    z = np.zeros((s_local, b, hd))
    h, _, _, _ = nm.sp_norm_fwd(z, np.ones_like(z), np.ones(hd), np.zeros(hd), norm="layernorm",
                                eps=1e-5, p_drop=p, seed=4, site=2, seq_offset=16)
    M = ph.hidden_keep_mask(4, p, 2, s_local, b, hd, 16)
    assert 0 < M.mean() < 1
    np.testing.assert_array_equal(h, M / (1 - p))


def test_dropout_forward_and_backward_equal_torch_with_constant_mask():
    resid, y, du, dres, gamma, beta = _inputs(5, 2, 24, seed=2)
    p, seed = 0.3, 8
    kw = dict(norm="layernorm", p_drop=p, seed=seed, site=1, seq_offset=7)
    h, u, mu, rstd = nm.sp_norm_fwd(resid, y, gamma, beta, eps=1e-5, **kw)
    M = torch.tensor(ph.hidden_keep_mask(seed, p, 1, 5, 2, 24, 7), dtype=torch.float64)
    tr = torch.tensor(resid, requires_grad=True)
    ty = torch.tensor(y, requires_grad=True)
    th = tr + ty * M / (1 - p)
    tu = F.layer_norm(th, (24,), torch.tensor(gamma), torch.tensor(beta), eps=1e-5)
    np.testing.assert_allclose(u, tu.detach().numpy(), rtol=1e-12, atol=1e-12)
    torch.autograd.backward([tu, th], [torch.tensor(du), torch.tensor(dres)])
    dh, dy, _, _ = nm.sp_norm_bwd(du, dres, h, gamma, mu, rstd, **kw)
    np.testing.assert_allclose(dh, tr.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dy, ty.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_layernorm_closed_forms():
    resid, y, du, dres, gamma, beta = _inputs(4, 2, 64, seed=3)
    eps = 1e-5
    h, u, mu, rstd = nm.sp_norm_fwd(resid, y, np.ones(64), np.zeros(64), norm="layernorm",
                                    eps=eps, p_drop=0.1, seed=0, site=1)
    var = h.var(axis=-1)
    np.testing.assert_allclose(u.mean(axis=-1), 0.0, atol=1e-13)
    np.testing.assert_allclose(u.var(axis=-1), var / (var + eps), rtol=1e-12)
    dh, _, _, _ = nm.sp_norm_bwd(du, dres, h, np.ones(64), mu, rstd, norm="layernorm",
                                 p_drop=0.1, seed=0, site=1)
    xhat = (h - mu[..., None]) * rstd[..., None]
    # LayerNorm's input gradient sums to zero over a row; against xhat it
    # leaves rstd * mean(g xhat) * (n - sum xhat^2), zero only when eps = 0
    np.testing.assert_allclose((dh - dres).sum(-1), 0.0, atol=1e-12)
    g = du
    want = rstd * (g * xhat).mean(-1) * (64 - (xhat * xhat).sum(-1))
    np.testing.assert_allclose(((dh - dres) * xhat).sum(-1), want, rtol=1e-6, atol=1e-12)


@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_finite_differences(norm):
    resid, y, du, dres, gamma, beta = _inputs(2, 2, 8, seed=4)
    kw = dict(norm=norm, p_drop=0.3, seed=6, site=1)
    h, u, mu, rstd = nm.sp_norm_fwd(resid, y, gamma, beta, eps=1e-5, **kw)
    dh, dy, dgamma, dbeta = nm.sp_norm_bwd(du, dres, h, gamma, mu, rstd, **kw)

    def loss(r, yy, g, bt):
        hh, uu, _, _ = nm.sp_norm_fwd(r, yy, g, bt, eps=1e-5, **kw)
        return (uu * du).sum() + (hh * dres).sum()

    eps = 1e-6
    for target, grad in ((0, dh), (1, dy), (2, dgamma), (3, dbeta)):
        if grad is None:
            continue
        args = [resid, y, gamma, beta]
        x = args[target]
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            a = [t.copy() for t in args]; a[target][idx] += eps
            m = [t.copy() for t in args]; m[target][idx] -= eps
            num[idx] = (loss(*a) - loss(*m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_sequence_split_invariance():
    """Ranks holding rows [0,8), [8,16) with seq_offset reproduce the unsplit run."""
    resid, y, du, dres, gamma, beta = _inputs(16, 2, 32, seed=5)
    kw = dict(norm="layernorm", p_drop=0.2, seed=3, site=2)
    h, u, mu, rstd = nm.sp_norm_fwd(resid, y, gamma, beta, eps=1e-5, **kw)
    g = nm.sp_norm_bwd(du, dres, h, gamma, mu, rstd, **kw)
    for lo in (0, 8):
        sl = slice(lo, lo + 8)
        hs, us, ms, rs = nm.sp_norm_fwd(resid[sl], y[sl], gamma, beta, eps=1e-5, seq_offset=lo, **kw)
        np.testing.assert_array_equal(hs, h[sl])
        np.testing.assert_array_equal(us, u[sl])
        gs = nm.sp_norm_bwd(du[sl], dres[sl], hs, gamma, ms, rs, seq_offset=lo, **kw)
        np.testing.assert_array_equal(gs[0], g[0][sl])
        np.testing.assert_array_equal(gs[1], g[1][sl])
