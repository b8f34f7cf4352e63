"""Graph capture: one step of the hot path (attention core forward and
backward, norm region forward and backward) captured into a HIP graph through
torch.cuda.graph, replayed several times with eager work and synchronisations
between the replays; every replay equals the eager step bit for bit.  The
library issues kernels only (no allocation, no memset), so it can be
captured."""
import pytest
import torch

from selective_recompute_attention_attn_amd import gen, ops
from gpu_util import announce, dev, need_gpu


def _step(t, a, n):
    akw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed)
    o, lse = ops.attn_core_fwd(t["q"], t["k"], t["v"], **akw)
    dq, dk, dv = ops.attn_core_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], **akw)
    nkw = dict(norm=n.norm, p_drop=n.p_drop, seed=n.seed, site=n.site)
    h, u, mean, rstd = ops.sp_norm_fwd(t["resid"], t["y"], t["gamma"], t["beta"], eps=n.eps, **nkw)
    dh, dy, dg, db = ops.sp_norm_bwd(t["du"], t["dres"], h, t["gamma"], mean, rstd, **nkw)
    return [o, lse, dq, dk, dv, h, u, mean, rstd, dh, dy, dg, db]


@pytest.mark.gpu
@pytest.mark.parametrize("d,hkv", [(64, 4), (128, 2)])
def test_captured_step_replays_equal_the_eager_step(d, hkv):
    device = need_gpu()
    a = gen.AttnShape(b=2, s=320, hq=4, hkv=hkv, d=d, causal=True, p_drop=0.1, seed=8)
    n = gen.NormShape(s_local=40, b=2, h=1024, norm="layernorm", p_drop=0.1, seed=8)
    announce(f"graph capture {a} {n}")
    xa, xn = gen.attn_inputs(a, seed_base=3), gen.norm_inputs(n, seed_base=3)
    t = {k: dev(xa[k], "bf16", device) for k in ("q", "k", "v", "do")}
    t.update({k: dev(xn[k], "bf16", device) for k in ("resid", "y", "du", "dres")})
    t["gamma"] = torch.tensor(xn["gamma"], device=device)
    t["beta"] = torch.tensor(xn["beta"], device=device)

    eager = [x.clone() for x in _step(t, a, n)]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(t, a, n)                      # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static = _step(t, a, n)
    for r in range(4):
        for x in static:
            x.fill_(float("nan") if x.is_floating_point() else 0)   # replays must overwrite
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(static, eager)):
            assert torch.equal(x, y), (r, i)
        _step(t, a, n)                      # eager work between the replays
        torch.cuda.synchronize()
