"""GPU parity of the sequence-parallel norm region (HIP, through the C ABI)
against the oracle: fp32 within 1e-5, bf16 within 2e-2 (max-norm relative per
tensor), hidden-dropout mask bit-exact."""
import numpy as np
import pytest
import torch

from oracle import norm as onm
from oracle import philox as oph
from selective_recompute_attention_attn_amd import gen, ops
from tests.gpu_util import TOL_BF16, TOL_FP32, announce, assert_close, dev, host, need_gpu

pytestmark = pytest.mark.gpu


def run_both(n: gen.NormShape, x, device, alias_dy=False):
    kw = dict(norm=n.norm, p_drop=n.p_drop, seed=n.seed, site=n.site, seq_offset=n.seq_offset)
    resid, y, du, dres = (dev(x[k], n.dtype, device) for k in ("resid", "y", "du", "dres"))
    gamma = torch.tensor(x["gamma"], device=device)
    beta = torch.tensor(x["beta"], device=device)
    h, u, mean, rstd = ops.sp_norm_fwd(resid, y, gamma, beta, eps=n.eps, **kw)
    dh, dy, dg, db = ops.sp_norm_bwd(du, dres, h, gamma, mean, rstd, alias_dy=alias_dy, **kw)
    torch.cuda.synchronize()
    got = dict(h=host(h), u=host(u), rstd=host(rstd), dh=host(dh), dy=host(dy), dgamma=host(dg))
    if n.norm == "layernorm":
        got["mean"] = host(mean)
        got["dbeta"] = host(db)
    rh, ru, rm, rr = onm.sp_norm_fwd(x["resid"], x["y"], x["gamma"], x["beta"], eps=n.eps, **kw)
    rdh, rdy, rdg, rdb = onm.sp_norm_bwd(x["du"], x["dres"], rh, x["gamma"], rm, rr, **kw)
    ref = dict(h=rh, u=ru, rstd=rr.reshape(-1), dh=rdh, dy=rdy, dgamma=rdg)
    if n.norm == "layernorm":
        ref["mean"] = rm.reshape(-1)
        ref["dbeta"] = rdb
    return got, ref


def check(got, ref, tol):
    """Per-tensor and per-row max-norm relative errors (rows of h values for h,
    u, dh, dy; one value per row for the statistics; dgamma and dbeta are
    per-column sums over all rows, checked per tensor).  A row's mean is a sum
    of terms h_j / h that can nearly cancel: it is judged against the larger of
    itself and mean |h_j|, the size of its terms."""
    def row_len(k):
        if k in ("mean", "rstd"):
            return 1
        return 0 if k in ("dgamma", "dbeta") else np.asarray(ref[k]).shape[-1]
    h_ref = np.asarray(ref["h"], np.float64)
    floors = {"mean": np.mean(np.abs(h_ref.reshape(-1, h_ref.shape[-1])), axis=1)}
    return {k: assert_close(k, got[k], ref[k], tol, row_len=row_len(k), row_floor=floors.get(k)) for k in ref}


def test_tiny_fp32_workload():
    device = need_gpu()
    n = gen.WORKLOADS["tiny-fp32"].norm
    announce(f"norm tiny-fp32 {n}")
    print(check(*run_both(n, gen.norm_inputs(n), device), TOL_FP32))


SHAPES = [
    # s_local, b, h, norm, p, dtype
    (7, 3, 200, "layernorm", 0.1, "bf16"),
    (64, 2, 6144, "layernorm", 0.1, "bf16"),
    (5, 1, 20480, "layernorm", 0.1, "bf16"),
    (33, 1, 8192, "rmsnorm", 0.0, "bf16"),
    (300, 2, 96, "layernorm", 0.3, "bf16"),
    (9, 2, 1000, "rmsnorm", 0.2, "fp32"),
    (600, 1, 64, "layernorm", 0.1, "fp32"),
    (1500, 2, 256, "layernorm", 0.1, "bf16"),      # several rows per workgroup, odd remainder
    (3, 1, 32768, "layernorm", 0.1, "bf16"),       # largest row: 4 groups per thread of 1024
    (2, 2, 28672, "rmsnorm", 0.0, "bf16"),
]


@pytest.mark.parametrize("s_local,b,h,norm,p,dtype", SHAPES)
def test_shapes(s_local, b, h, norm, p, dtype):
    device = need_gpu()
    n = gen.NormShape(s_local=s_local, b=b, h=h, norm=norm, p_drop=p, dtype=dtype, seed=11, site=2,
                      seq_offset=40, gamma="u0.9-1.1", beta="n0.02" if norm == "layernorm" else "zeros")
    announce(f"norm {n}")
    print(check(*run_both(n, gen.norm_inputs(n, seed_base=3), device), TOL_BF16 if dtype == "bf16" else TOL_FP32))


def test_dy_aliases_dh_without_dropout():
    device = need_gpu()
    n = gen.NormShape(s_local=16, b=2, h=512, norm="rmsnorm", p_drop=0.0)
    announce("norm alias dy")
    got, ref = run_both(n, gen.norm_inputs(n), device, alias_dy=True)
    check(got, ref, TOL_BF16)


def test_hidden_mask_bit_exact_and_visible():
    device = need_gpu()
    s_local, b, h, p, seed, site, off = 24, 3, 200, 0.1, 77, 2, 1000
    announce("hidden mask")
    m = ops.hidden_dropout_mask(s_local, b, h, p_drop=p, seed=seed, site=site, seq_offset=off, device=device)
    ref = oph.hidden_keep_mask(seed, p, site, s_local, b, h, off)
    np.testing.assert_array_equal(m.cpu().numpy().astype(bool), ref)
    # black box: resid = 0, y = 1 gives h = M / (1 - p) exactly in fp32
    z = torch.zeros((s_local, b, h), device=device)
    hh, _, _, _ = ops.sp_norm_fwd(z, torch.ones_like(z), torch.ones(h, device=device), torch.zeros(h, device=device),
                                  p_drop=p, seed=seed, site=site, seq_offset=off)
    inv_keep = np.float32(1.0) / (np.float32(1.0) - np.float32(p))
    np.testing.assert_array_equal(hh.cpu().numpy(), np.where(ref, inv_keep, np.float32(0.0)))


def test_sequence_split_invariance():
    device = need_gpu()
    n = gen.NormShape(s_local=64, b=2, h=1024, norm="layernorm", p_drop=0.2, seed=5)
    announce("norm split invariance")
    x = gen.norm_inputs(n)
    full, _ = run_both(n, x, device)
    for lo in (0, 32):
        sub = {k: (v[lo:lo + 32] if v.ndim == 3 else v) for k, v in x.items()}
        part, _ = run_both(n.with_(s_local=32, seq_offset=lo), sub, device)
        for k in ("h", "u", "dh", "dy"):
            np.testing.assert_array_equal(part[k], full[k][lo:lo + 32])


@pytest.mark.parametrize("name", ["gpt22b-t8", "gpt175b-t8", "gpt530b-t8", "llama3-70b-t8"])
def test_full_size_workload(name):
    device = need_gpu()
    n = gen.WORKLOADS[name].norm
    announce(f"norm full-size {name}")
    got, ref = run_both(n, gen.norm_inputs(n), device, alias_dy=n.p_drop == 0.0)
    print(name, check(got, ref, TOL_BF16))


def test_empty_rows_give_zero_parameter_grads():
    device = need_gpu()
    announce("norm empty rows")
    h = 512
    z = torch.empty((0, 2, h), dtype=torch.bfloat16, device=device)
    gamma = torch.ones(h, device=device)
    mean = torch.empty(0, device=device)
    rstd = torch.empty(0, device=device)
    dg = torch.full((h,), 7.0, device=device)
    db = torch.full((h,), 7.0, device=device)
    ops.sp_norm_bwd(z, z, z, gamma, mean, rstd, p_drop=0.1, outs=(z, torch.empty_like(z), dg, db))
    torch.cuda.synchronize()
    assert not dg.any() and not db.any()


def test_parameter_grads_are_reproducible():
    device = need_gpu()
    n = gen.NormShape(s_local=256, b=4, h=6144, norm="layernorm", p_drop=0.1, seed=9)
    announce("norm determinism")
    x = gen.norm_inputs(n)
    a, _ = run_both(n, x, device)
    b, _ = run_both(n, x, device)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
