"""The layer around the attention core (layer.py) on the GPU against the
oracle's float64 layer, and full recomputation against selective."""

import numpy as np
import pytest
import torch

from oracle import layer as ol
from selective_recompute_attention_attn_amd import layer as gl
from gpu_util import announce, need_gpu

TOL_BF16 = 2e-2


def _rel(x, ref):
    x = x.detach().float().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-30))


@pytest.mark.gpu
@pytest.mark.parametrize("s,b,h,hq,d,ffn,causal,p", [
    (96, 2, 128, 2, 64, 256, True, 0.1),
    (96, 2, 128, 2, 64, 256, False, 0.0),
    # d = 128: the two-group forward and dQ kernels and the producer/consumer
    # dK/dV kernel, three 128-query tiles (the longest split), 8 heads
    (384, 1, 1024, 8, 128, 2048, True, 0.1),
    (384, 1, 1024, 8, 128, 2048, True, 0.0),
])
def test_layer_matches_oracle(s, b, h, hq, d, ffn, causal, p):
    device = need_gpu()
    announce(f"layer s={s} b={b} h={h} hq={hq} d={d} ffn={ffn} causal={causal} p={p}")
    w = gl.random_weights(h, hq, d, ffn, device=device, seed=4)
    layer = gl.Layer(w, hq=hq, d=d, causal=causal, p_attn=p, p_hidden=p, seed=9)
    g = torch.Generator().manual_seed(5)
    x = torch.randn(s, b, h, generator=g).to(torch.bfloat16)
    dh2 = torch.randn(s, b, h, generator=g).to(torch.bfloat16)
    du3 = torch.randn(s, b, h, generator=g).to(torch.bfloat16)
    xg = x.to(device).requires_grad_(True)
    h2, u3 = layer(xg)
    torch.autograd.backward((h2, u3), (dh2.to(device), du3.to(device)))
    torch.cuda.synchronize()

    wn = {k: v.detach().float().cpu().numpy().astype(np.float64) for k, v in w.items()}
    cfg = dict(hq=hq, d=d, causal=causal, p_attn=p, p_hidden=p, seed=9, eps=1e-5)
    f64 = lambda t: t.float().numpy().astype(np.float64)
    rh2, ru3, cache = ol.layer_fwd(f64(x), wn, cfg)
    rdx, rg = ol.layer_bwd(f64(dh2), f64(du3), wn, cfg, cache)
    errs = {"h2": _rel(h2, rh2), "u3": _rel(u3, ru3), "dx": _rel(xg.grad, rdx)}
    errs.update({k: _rel(w[k].grad, rg[k]) for k in ol.WEIGHTS})
    print({k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= TOL_BF16}
    assert not bad, bad


@pytest.mark.gpu
def test_full_recompute_gives_the_selective_gradients():
    """Full recomputation re-runs the layer's forward pass in the backward pass;
    the masks are functions of position and seed, so every gradient is the same
    as under selective recomputation, bit for bit."""
    device = need_gpu()
    s, b, h, hq, d, ffn = 128, 2, 192, 2, 96, 384
    announce("layer full vs selective recompute")
    g = torch.Generator().manual_seed(6)
    x = torch.randn(s, b, h, generator=g).to(torch.bfloat16).to(device)
    dys = [torch.randn(s, b, h, generator=g).to(torch.bfloat16).to(device) for _ in range(2)]
    grads = {}
    for mode in ("selective", "full"):
        w = gl.random_weights(h, hq, d, ffn, device=device, seed=7)
        layer = gl.Layer(w, hq=hq, d=d, causal=True, p_attn=0.1, p_hidden=0.1, seed=3)
        xg = x.clone().requires_grad_(True)
        torch.autograd.backward(layer(xg, mode), dys)
        torch.cuda.synchronize()
        grads[mode] = [xg.grad] + [w[k].grad for k in gl.Layer.WEIGHTS]
    for a, c in zip(grads["selective"], grads["full"]):
        assert torch.equal(a, c)
