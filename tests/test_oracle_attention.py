"""Pins for the oracle's attention core.

Each test fixes the oracle to something other than itself: torch's
scaled_dot_product_attention (a library routine, CPU float64), torch
autograd, scipy's logsumexp, closed forms, central finite differences, and
the Philox mask pinned to rocRAND in test_oracle_philox.
"""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import attention as at
from oracle import philox as ph


def _inputs(b, s, hq, hkv, d, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, s, hq, d)) * scale
    k = rng.standard_normal((b, s, hkv, d)) * scale
    v = rng.standard_normal((b, s, hkv, d)) * scale
    do = rng.standard_normal((b, s, hq, d)) * scale
    return q, k, v, do


def _sdpa(q, k, v, causal, scale):
    """torch SDPA (math path, CPU, float64) in the [b, s, h, d] layout."""
    grp = q.shape[2] // k.shape[2]
    tq = torch.tensor(q).permute(0, 2, 1, 3)
    tk = torch.tensor(k).permute(0, 2, 1, 3).repeat_interleave(grp, dim=1)
    tv = torch.tensor(v).permute(0, 2, 1, 3).repeat_interleave(grp, dim=1)
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one_and_lse(causal):
    q, k, _, _ = _inputs(1, 96, 2, 2, 16)
    scale = 1 / np.sqrt(16)
    P, lse = at.attn_probs(q, k, causal=causal, scale=scale, bb=0, hh=1)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    S = at.scores(q[0, :, 1], k[0, :, 1], scale, causal)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(S, axis=1), rtol=1e-13)
    np.testing.assert_allclose(np.exp(S - lse[:, None]), P, atol=1e-15)
    if causal:
        assert np.all(P[np.triu_indices(96, 1)] == 0)


@pytest.mark.parametrize("causal,hq,hkv", [(False, 2, 2), (True, 4, 4), (True, 4, 1), (False, 6, 2)])
def test_fwd_p0_equals_sdpa(causal, hq, hkv):
    q, k, v, _ = _inputs(2, 80, hq, hkv, 24, seed=1)
    scale = 1 / np.sqrt(24)
    O, lse = at.attn_fwd(q, k, v, causal=causal, scale=scale, p_drop=0.0, seed=0)
    np.testing.assert_allclose(O, _sdpa(q, k, v, causal, scale), rtol=1e-12, atol=1e-12)


def test_fwd_dropout_composition_identity_v():
    """V = I (d = s) makes O = P_d itself: it must equal SDPA's P times M/(1-p)."""
    s, p, seed = 32, 0.3, 77
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, s, 1, s))
    k = rng.standard_normal((1, s, 1, s))
    v = np.eye(s)[None, :, None, :]
    scale = 0.2
    O, _ = at.attn_fwd(q, k, v, causal=True, scale=scale, p_drop=p, seed=seed, head_offset=5)
    P = _sdpa(q, k, v, True, scale)[0, :, 0]           # p = 0, V = I -> P
    M = ph.attn_keep_mask(seed, p, 0, 5, s, s)
    assert 0 < M.mean() < 1
    np.testing.assert_allclose(O[0, :, 0], P * M / (1 - p), rtol=1e-12, atol=1e-14)


def test_closed_forms():
    s, d, p, seed = 48, 8, 0.25, 3
    q, k, v, _ = _inputs(1, s, 1, 1, d, seed=4)
    # causal row 0 sees only key 0: O_0 = V_0 * M_00 / (1 - p)
    O, lse = at.attn_fwd(q, k, v, causal=True, scale=0.3, p_drop=p, seed=seed)
    M = ph.attn_keep_mask(seed, p, 0, 0, s, s)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0] * M[0, 0] / (1 - p), rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0, 0], q[0, 0, 0] @ k[0, 0, 0] * 0.3, rtol=1e-14)
    # Q = 0: every visible score is 0, so P_ij = 1/n_i
    qz = np.zeros_like(q)
    O, lse = at.attn_fwd(qz, k, v, causal=True, scale=0.3, p_drop=p, seed=seed)
    n = np.arange(1, s + 1)
    want = np.array([(M[i, :i + 1, None] * v[0, :i + 1, 0]).sum(0) / ((1 - p) * n[i]) for i in range(s)])
    np.testing.assert_allclose(O[0, :, 0], want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(n), rtol=1e-14)


@pytest.mark.parametrize("causal,hq,hkv", [(True, 2, 2), (False, 4, 2), (True, 4, 1)])
def test_bwd_p0_equals_torch_autograd(causal, hq, hkv):
    q, k, v, do = _inputs(2, 40, hq, hkv, 16, seed=5)
    scale = 1 / np.sqrt(16)
    O, lse = at.attn_fwd(q, k, v, causal=causal, scale=scale, p_drop=0.0, seed=0)
    dq, dk, dv = at.attn_bwd(q, k, v, lse, do, causal=causal, scale=scale, p_drop=0.0, seed=0)
    grp = hq // hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    o = F.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(grp, 1),
        tv.permute(0, 2, 1, 3).repeat_interleave(grp, 1), is_causal=causal, scale=scale)
    o.permute(0, 2, 1, 3).backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_bwd_dropout_equals_torch_autograd_with_constant_mask():
    """Autograd differentiates softmax + masked product; the mask is a constant."""
    b, s, hq, hkv, d, p, seed = 1, 24, 2, 1, 8, 0.3, 11
    q, k, v, do = _inputs(b, s, hq, hkv, d, seed=6)
    scale = 0.35
    O, lse = at.attn_fwd(q, k, v, causal=True, scale=scale, p_drop=p, seed=seed, head_offset=3)
    dq, dk, dv = at.attn_bwd(q, k, v, lse, do, causal=True, scale=scale, p_drop=p, seed=seed,
                             head_offset=3)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    causal = torch.ones(s, s, dtype=torch.bool).tril()
    outs = []
    for hh in range(hq):
        S = tq[0, :, hh] @ tk[0, :, 0].T * scale
        P = torch.softmax(S.masked_fill(~causal, float("-inf")), dim=-1)
        M = torch.tensor(ph.attn_keep_mask(seed, p, 0, 3 + hh, s, s), dtype=torch.float64)
        outs.append((P * M / (1 - p)) @ tv[0, :, 0])
    o = torch.stack(outs, dim=1)[None]
    np.testing.assert_allclose(O, o.detach().numpy(), rtol=1e-12, atol=1e-13)
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_bwd_finite_differences_fixed_mask():
    """Central differences of L = sum(O * dO): smooth in q, k, v for a fixed seed."""
    b, s, hq, hkv, d, p, seed = 1, 8, 2, 1, 4, 0.3, 21
    q, k, v, do = _inputs(b, s, hq, hkv, d, seed=8)
    kw = dict(causal=True, scale=0.5, p_drop=p, seed=seed)
    O, lse = at.attn_fwd(q, k, v, **kw)
    grads = at.attn_bwd(q, k, v, lse, do, **kw)
    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p = [q, k, v]; args_p[which] = xp
            args_m = [q, k, v]; args_m[which] = xm
            lp = (at.attn_fwd(*args_p, **kw)[0] * do).sum()
            lm = (at.attn_fwd(*args_m, **kw)[0] * do).sum()
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grads[which], num, rtol=1e-6, atol=1e-8)


def test_bwd_identity_rowsum_do_o_equals_rowsum_dp_p():
    q, k, v, do = _inputs(1, 64, 1, 1, 16, seed=9)
    p, seed, scale = 0.2, 5, 0.25
    O, lse = at.attn_fwd(q, k, v, causal=True, scale=scale, p_drop=p, seed=seed)
    P, _ = at.attn_probs(q, k, causal=True, scale=scale, bb=0, hh=0)
    M = ph.attn_keep_mask(seed, p, 0, 0, 64, 64)
    dP = (do[0, :, 0] @ v[0, :, 0].T) * M / (1 - p)
    np.testing.assert_allclose((do[0, :, 0] * O[0, :, 0]).sum(1), (dP * P).sum(1), rtol=1e-11)


def test_store_and_recompute_give_the_same_gradients():
    q, k, v, do = _inputs(1, 64, 2, 2, 16, seed=10)
    p, seed, scale = 0.1, 0, 0.25
    O, lse = at.attn_fwd(q, k, v, causal=False, scale=scale, p_drop=p, seed=seed)
    dq, dk, dv = at.attn_bwd(q, k, v, lse, do, causal=False, scale=scale, p_drop=p, seed=seed)
    for hh in range(2):
        P, _ = at.attn_probs(q, k, causal=False, scale=scale, bb=0, hh=hh)
        M = ph.attn_keep_mask(seed, p, 0, hh, 64, 64)   # the forward's mask, stored
        sq, sk, sv = at.attn_bwd_stored(P, M, q[0, :, hh], k[0, :, hh], v[0, :, hh],
                                        do[0, :, hh], scale=scale, p_drop=p)
        np.testing.assert_allclose(dq[0, :, hh], sq, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dk[0, :, hh], sk, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dv[0, :, hh], sv, rtol=1e-12, atol=1e-13)


def test_head_offset_split_invariance():
    """Two ranks holding heads [0, 2) and [2, 4) reproduce the 4-head run."""
    q, k, v, do = _inputs(1, 32, 4, 4, 8, seed=12)
    kw = dict(causal=True, scale=0.3, p_drop=0.2, seed=9)
    O, lse = at.attn_fwd(q, k, v, **kw)
    g = at.attn_bwd(q, k, v, lse, do, **kw)
    for lo in (0, 2):
        sl = slice(lo, lo + 2)
        Os, ls = at.attn_fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], head_offset=lo, **kw)
        gs = at.attn_bwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], ls, do[:, :, sl],
                         head_offset=lo, **kw)
        np.testing.assert_array_equal(Os, O[:, :, sl])
        for a, bfull in zip(gs, g):
            np.testing.assert_array_equal(a, bfull[:, :, sl])


def test_heads_subset_matches_full():
    q, k, v, do = _inputs(2, 32, 4, 2, 8, seed=13)
    kw = dict(causal=True, scale=0.3, p_drop=0.1, seed=1)
    O, lse = at.attn_fwd(q, k, v, **kw)
    Os, ls = at.attn_fwd(q, k, v, heads=[(1, 3)], **kw)
    np.testing.assert_array_equal(Os[1, :, 3], O[1, :, 3])
    np.testing.assert_array_equal(ls[1, 3], lse[1, 3])


def _sdpa_padded(q, k, v, do, lens, causal, scale):
    """torch SDPA (CPU, float64) with a key-padding (and causal) boolean mask;
    dO of padded query rows is zeroed so that they contribute nothing."""
    b, s, hq, _ = q.shape
    grp = hq // k.shape[2]
    allow = np.zeros((b, 1, s, s), dtype=bool)
    for bb, L in enumerate(lens):
        allow[bb, 0, :, :L] = True
    if causal:
        allow &= np.tril(np.ones((s, s), dtype=bool))[None, None]
    allow[:, :, :, 0] |= ~allow.any(axis=3)      # rows with no visible key: any finite output, discarded
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    o = F.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(grp, 1),
        tv.permute(0, 2, 1, 3).repeat_interleave(grp, 1), attn_mask=torch.tensor(allow), scale=scale)
    gdo = do.copy()
    for bb, L in enumerate(lens):
        gdo[bb, L:] = 0.0
    o.permute(0, 2, 1, 3).backward(torch.tensor(gdo))
    return o.permute(0, 2, 1, 3).detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal,hq,hkv", [(True, 2, 2), (False, 4, 2), (True, 4, 1)])
def test_padded_batch_p0_equals_masked_sdpa(causal, hq, hkv):
    """Padded batch, p = 0: valid rows equal torch SDPA with a key-padding
    mask (forward and autograd backward); padded rows are zero, LSE -inf."""
    lens = [37, 0, 50, 12]
    q, k, v, do = _inputs(4, 50, hq, hkv, 16, seed=9)
    scale = 1 / np.sqrt(16)
    O, lse = at.attn_fwd(q, k, v, causal=causal, scale=scale, p_drop=0.0, seed=0, seqlens=lens)
    dq, dk, dv = at.attn_bwd(q, k, v, lse, do, causal=causal, scale=scale, p_drop=0.0, seed=0, seqlens=lens)
    o_ref, dq_ref, dk_ref, dv_ref = _sdpa_padded(q, k, v, do, lens, causal, scale)
    for bb, L in enumerate(lens):
        np.testing.assert_allclose(O[bb, :L], o_ref[bb, :L], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dq[bb, :L], dq_ref[bb, :L], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk[bb], dk_ref[bb], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv[bb], dv_ref[bb], rtol=1e-10, atol=1e-12)
        assert not O[bb, L:].any() and not dq[bb, L:].any()
        assert not dk[bb, L:].any() and not dv[bb, L:].any()
        assert np.all(np.isneginf(lse[bb, :, L:]))


def test_padded_batch_with_dropout_equals_truncated_sequences():
    """With dropout, each element of a padded batch equals the same element
    run alone at its valid length: the mask keeps its global counters."""
    lens = [33, 64, 1]
    q, k, v, do = _inputs(3, 64, 2, 1, 16, seed=10)
    kw = dict(causal=True, scale=0.25, p_drop=0.2, seed=77, head_offset=3)
    O, lse = at.attn_fwd(q, k, v, seqlens=lens, **kw)
    dq, dk, dv = at.attn_bwd(q, k, v, lse, do, seqlens=lens, **kw)
    for bb, L in enumerate(lens):
        # batch index bb enters the counters: run the element at its own index
        sl = lambda x: x[: bb + 1, :L]
        O1, lse1 = at.attn_fwd(sl(q), sl(k), sl(v), heads=[(bb, h) for h in range(2)], **kw)
        dq1, dk1, dv1 = at.attn_bwd(sl(q), sl(k), sl(v), lse1, sl(do), heads=[(bb, h) for h in range(2)], **kw)
        np.testing.assert_array_equal(O[bb, :L], O1[bb])
        np.testing.assert_array_equal(lse[bb, :, :L], lse1[bb])
        np.testing.assert_array_equal(dq[bb, :L], dq1[bb])
        np.testing.assert_array_equal(dk[bb, :L], dk1[bb])
        np.testing.assert_array_equal(dv[bb, :L], dv1[bb])
