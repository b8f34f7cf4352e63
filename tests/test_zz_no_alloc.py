"""The allocation-free backward (srat_attn_core_bwd_noalloc, through the C ABI)
against srat_attn_core_bwd on the same inputs: bit for bit equal, on calls in a
row that reuse the library's scratch with shrinking shapes (the second and
third call see what the previous one left there).  The reference call's
workspace is filled with 0xFF bytes (NaN patterns) first, so a kernel reading
a workspace byte it has not written would show up as a mismatch."""
import numpy as np
import pytest
import torch

from selective_recompute_attention_attn_amd import gen, ops
from tests.gpu_util import announce, dev, need_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # b, s, hq, hkv, d, causal, p: grouped-query partials, then a split grid, then a plain one
    (1, 2048, 8, 1, 128, True, 0.0),
    (1, 384, 4, 2, 128, True, 0.1),
    (2, 130, 2, 2, 64, True, 0.1),
]


def _inputs(a, device):
    x = gen.attn_inputs(a, seed_base=23)
    q, k, v, do = (dev(x[n], "bf16", device) for n in ("q", "k", "v", "do"))
    kw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed, head_offset=a.head_offset)
    o, lse = ops.attn_core_fwd(q, k, v, **kw)
    return q, k, v, do, o, lse, kw


def test_noalloc_backward_equals_the_workspace_backward():
    device = need_gpu()
    for b, s, hq, hkv, d, causal, p in CASES:
        a = gen.AttnShape(b=b, s=s, hq=hq, hkv=hkv, d=d, causal=causal, p_drop=p, seed=77, head_offset=2)
        announce(f"no-alloc backward {a}")
        q, k, v, do, o, lse, kw = _inputs(a, device)
        desc = ops.attn_desc(q, k, v, o, **kw)
        ws = torch.full((max(ops.attn_bwd_workspace_bytes(desc), 1),), 0xFF, dtype=torch.uint8, device=device)
        ref = ops.attn_core_bwd(q, k, v, o, lse, do, workspace=ws, **kw)
        got = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
        ops.attn_core_bwd_noalloc(q, k, v, o, lse, do, *got, **kw)
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.isfinite(r.float()).all(), name
            np.testing.assert_array_equal(g.float().cpu().numpy(), r.float().cpu().numpy(), err_msg=name)


def test_noalloc_backward_allocates_nothing():
    """No device memory is allocated through torch during the call, and the
    call refuses a shape whose workspace exceeds the scratch."""
    device = need_gpu()
    a = gen.AttnShape(b=1, s=512, hq=4, hkv=1, d=128, causal=True, p_drop=0.1, seed=5)
    announce("no-alloc backward, allocation check")
    q, k, v, do, o, lse, kw = _inputs(a, device)
    grads = tuple(torch.empty_like(t) for t in (q, k, v))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(device)
    torch.cuda.reset_peak_memory_stats(device)
    ops.attn_core_bwd_noalloc(q, k, v, o, lse, do, *grads, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated(device) == before
    big = gen.AttnShape(b=1, s=32768, hq=8, hkv=1, d=128, causal=True, p_drop=0.0)
    qb = torch.empty((big.b, big.s, big.hq, big.d), dtype=torch.bfloat16, device=device)
    kb = torch.empty((big.b, big.s, big.hkv, big.d), dtype=torch.bfloat16, device=device)
    lb = torch.empty((big.b, big.hq, big.s), dtype=torch.float32, device=device)
    with pytest.raises(ops.SratError, match="SRAT_ERR_UNSUPPORTED"):
        ops.attn_core_bwd_noalloc(qb, kb, kb, qb, lb, qb, torch.empty_like(qb), torch.empty_like(kb),
                                  torch.empty_like(kb), causal=True)
