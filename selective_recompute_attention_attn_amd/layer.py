"""One transformer layer around the attention core, on one GPU.

The steps either side of the core as one tensor-parallel rank computes them,
without the collectives: LN1 -> QKV GEMM -> attention core -> output GEMM ->
hidden dropout + residual + LN2 -> MLP (exact GeLU) -> hidden dropout +
residual + LN3.  The attention core and the three norm regions are this
library's kernels (through ops); the four GEMMs and the GeLU are PyTorch's
(hipBLASLt), plain library GEMMs.

Two recompute policies ("Recomputing Activations" plate, second and third
paragraphs; LIT-736 record, Key takeaways bullet 4):
  * selective -- the attention core stores only O and its LSE, and its
    backward pass recomputes scores, softmax and dropout mask (what the
    library's attention calls do);
  * full      -- only the layer input is kept; the backward pass re-runs the
    layer's forward pass first (torch.utils.checkpoint).  Every mask is a
    function of its position and seed, so the re-run reproduces the forward
    pass exactly and both policies give the same gradients.

    python -m selective_recompute_attention_attn_amd.layer [--workload gpt22b-t8]

times the layer's forward and forward + backward under both policies and
prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import sys
from typing import Dict, Tuple

import torch
import torch.nn.functional as F
from torch.utils.checkpoint import checkpoint

from . import ops


class _AttnCore(torch.autograd.Function):
    """Attention core on the fused QKV GEMM output [s*b, 3*hq*d] (columns
    [q | k | v], head-major); returns O as [s*b, hq*d] for the output GEMM.
    Keeps q, k, v, O and the LSE; the backward pass recomputes the rest."""

    @staticmethod
    def forward(ctx, qkv, s, b, hq, d, causal, p_drop, seed):
        hd = hq * d
        heads = qkv.view(s, b, 3, hq, d)
        q, k, v = (heads[:, :, i].permute(1, 0, 2, 3) for i in range(3))
        obuf = torch.empty((s, b, hq, d), dtype=qkv.dtype, device=qkv.device)
        o = obuf.permute(1, 0, 2, 3)
        kw = dict(causal=causal, scale=1.0 / math.sqrt(d), p_drop=p_drop, seed=seed)
        _, lse = ops.attn_core_fwd(q, k, v, out=o, **kw)
        ctx.save_for_backward(qkv, obuf, lse)
        ctx.dims = (s, b, hq, d)
        ctx.kw = kw
        return obuf.view(s * b, hd)

    @staticmethod
    def backward(ctx, do2):
        qkv, obuf, lse = ctx.saved_tensors
        s, b, hq, d = ctx.dims
        heads = qkv.view(s, b, 3, hq, d)
        q, k, v = (heads[:, :, i].permute(1, 0, 2, 3) for i in range(3))
        o = obuf.permute(1, 0, 2, 3)
        do = do2.contiguous().view(s, b, hq, d).permute(1, 0, 2, 3)
        dqkv = torch.empty_like(qkv)
        dheads = dqkv.view(s, b, 3, hq, d)
        outs = tuple(dheads[:, :, i].permute(1, 0, 2, 3) for i in range(3))
        ops.attn_core_bwd(q, k, v, o, lse, do, outs=outs, **ctx.kw)
        return dqkv, None, None, None, None, None, None, None


class _Region(torch.autograd.Function):
    """Hidden dropout + residual + LayerNorm over [s, b, h] rows: (h, u)."""

    @staticmethod
    def forward(ctx, resid, y, gamma, beta, eps, p_drop, seed, site):
        h, u, mean, rstd = ops.sp_norm_fwd(resid, y, gamma, beta, norm="layernorm", eps=eps, p_drop=p_drop,
                                           seed=seed, site=site)
        ctx.save_for_backward(h, gamma, mean, rstd)
        ctx.kw = dict(norm="layernorm", p_drop=p_drop, seed=seed, site=site)
        return h, u

    @staticmethod
    def backward(ctx, dh_out, du):
        h, gamma, mean, rstd = ctx.saved_tensors
        dres = torch.zeros_like(h) if dh_out is None else dh_out.contiguous()
        du = torch.zeros_like(h) if du is None else du.contiguous()
        dh, dy, dg, db = ops.sp_norm_bwd(du, dres, h, gamma, mean, rstd, **ctx.kw)
        return dh, dy, dg, db, None, None, None, None


class Layer:
    """Weights of one layer (one tensor-parallel rank's share: hq heads of d,
    an MLP of width ffn) and its forward pass."""

    WEIGHTS = ("gamma1", "beta1", "w_qkv", "w_o", "gamma2", "beta2", "w_1", "w_2", "gamma3", "beta3")

    def __init__(self, weights: Dict[str, torch.Tensor], *, hq: int, d: int, causal: bool = True,
                 p_attn: float = 0.0, p_hidden: float = 0.0, seed: int = 0, eps: float = 1e-5):
        self.w = weights
        self.hq, self.d = hq, d
        self.causal, self.p_attn, self.p_hidden, self.seed, self.eps = causal, p_attn, p_hidden, seed, eps

    def forward(self, x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        """x: [s, b, h] (contiguous).  Returns (h2, u3)."""
        s, b, h = x.shape
        w = self.w
        _, u1 = _Region.apply(x, torch.zeros_like(x), w["gamma1"], w["beta1"], self.eps, 0.0, self.seed, 0)
        qkv = u1.view(s * b, h) @ w["w_qkv"]
        o2 = _AttnCore.apply(qkv, s, b, self.hq, self.d, self.causal, self.p_attn, self.seed)
        a = (o2 @ w["w_o"]).view(s, b, h)
        h1, u2 = _Region.apply(x, a, w["gamma2"], w["beta2"], self.eps, self.p_hidden, self.seed, 1)
        m = (F.gelu(u2.view(s * b, h) @ w["w_1"]) @ w["w_2"]).view(s, b, h)
        h2, u3 = _Region.apply(h1, m, w["gamma3"], w["beta3"], self.eps, self.p_hidden, self.seed, 2)
        return h2, u3

    def __call__(self, x: torch.Tensor, recompute: str = "selective"):
        if recompute == "selective":
            return self.forward(x)
        if recompute == "full":
            return checkpoint(self.forward, x, use_reentrant=False)
        raise ValueError(f"recompute must be 'selective' or 'full', not {recompute!r}")


def random_weights(h: int, hq: int, d: int, ffn: int, *, device, seed: int = 0, dtype=torch.bfloat16):
    """Seeded random weights (no trained weights exist for this path)."""
    g = torch.Generator().manual_seed(seed)
    hd = hq * d
    r = lambda *shape, std: (torch.randn(*shape, generator=g) * std)
    w = {"gamma1": 1 + 0.1 * torch.rand(h, generator=g), "beta1": r(h, std=0.02),
         "w_qkv": r(h, 3 * hd, std=1 / math.sqrt(h)), "w_o": r(hd, h, std=1 / math.sqrt(hd)),
         "gamma2": 1 + 0.1 * torch.rand(h, generator=g), "beta2": r(h, std=0.02),
         "w_1": r(h, ffn, std=1 / math.sqrt(h)), "w_2": r(ffn, h, std=1 / math.sqrt(ffn)),
         "gamma3": 1 + 0.1 * torch.rand(h, generator=g), "beta3": r(h, std=0.02)}
    out = {}
    for k, v in w.items():
        t = v.to(torch.float32 if k.startswith(("gamma", "beta")) else dtype).to(device)
        out[k] = t.requires_grad_(True)
    return out


def _bench(workload: str, steps: int, warmup: int) -> dict:
    from . import gen
    dev = torch.device("cuda:0")
    wl = gen.WORKLOADS[workload]
    a, n = wl.attn, wl.norm
    if a.hq != a.hkv or a.dtype != "bf16":
        raise SystemExit("the layer is built for bf16 multi-head attention (hq == hkv)")
    t = 8                          # the named workloads are one rank's share at t = 8
    h = n.h
    ffn = 4 * h // t
    weights = random_weights(h, a.hq, a.d, ffn, device=dev)
    layer = Layer(weights, hq=a.hq, d=a.d, causal=a.causal, p_attn=a.p_drop, p_hidden=n.p_drop, seed=1)
    g = torch.Generator().manual_seed(2)
    xs = [torch.randn(a.s, a.b, h, generator=g).to(torch.bfloat16).to(dev).requires_grad_(True) for _ in range(2)]
    dys = [torch.randn(a.s, a.b, h, generator=g).to(torch.bfloat16).to(dev) for _ in range(2)]

    def fwd(i, mode):
        with torch.no_grad():
            layer(xs[i % 2], mode)

    def fwd_bwd(i, mode):
        h2, u3 = layer(xs[i % 2], mode)
        torch.autograd.backward((h2, u3), (dys[i % 2], dys[(i + 1) % 2]))

    def timed(fn, mode):
        for i in range(warmup):
            fn(i, mode)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i, mode)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    res = {"workload": workload, "layer": {"s": a.s, "b": a.b, "h": h, "hq": a.hq, "d": a.d, "ffn": ffn,
                                           "tensor_parallel_share": t, "p_attn": a.p_drop, "p_hidden": n.p_drop},
           "steps": steps, "warmup": warmup}
    res["fwd_ms"] = timed(fwd, "selective")
    res["fwd_bwd_selective_ms"] = timed(fwd_bwd, "selective")
    res["fwd_bwd_full_ms"] = timed(fwd_bwd, "full")
    res["full_over_selective"] = res["fwd_bwd_full_ms"] / res["fwd_bwd_selective_ms"] - 1.0
    # the attention core's own forward, run alone on the layer's q, k, v: the
    # work selective recomputation re-does inside the core's backward
    with torch.no_grad():
        u1 = torch.randn(a.s * a.b, 3 * a.hq * a.d, generator=g).to(torch.bfloat16).to(dev)
        res["attn_core_fwd_ms"] = timed(lambda i, m: _AttnCore.apply(u1, a.s, a.b, a.hq, a.d, a.causal,
                                                                       a.p_drop, 1), None)
    res["selective_recompute_share"] = res["attn_core_fwd_ms"] / res["fwd_bwd_selective_ms"]
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="gpt22b-t8")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    print(json.dumps(_bench(args.workload, args.steps, args.warmup)), flush=True)


if __name__ == "__main__":
    main()
