"""GPU parity of the attention core (HIP, through the C ABI) against the oracle.

Same seeded inputs on both sides; fp32 path within 1e-5 and bf16 path within
2e-2 (max-norm relative error per tensor) of the float64 oracle; dropout
masks bit-exact.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oat
from oracle import philox as oph
from selective_recompute_attention_attn_amd import gen, ops
from tests.gpu_util import (TOL_BF16, TOL_FP32, announce, assert_close, dev, elementwise_err, grad_term_scales,
                            host, need_gpu)

pytestmark = pytest.mark.gpu


def run_gpu(a: gen.AttnShape, x, device):
    q, k, v, do = (dev(x[n], a.dtype, device) for n in ("q", "k", "v", "do"))
    kw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed, head_offset=a.head_offset)
    o, lse = ops.attn_core_fwd(q, k, v, **kw)
    dq, dk, dv = ops.attn_core_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    return {"o": host(o), "lse": host(lse), "dq": host(dq), "dk": host(dk), "dv": host(dv)}


def run_oracle(a: gen.AttnShape, x, heads=None):
    kw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed, head_offset=a.head_offset)
    o, lse = oat.attn_fwd(x["q"], x["k"], x["v"], heads=heads, **kw)
    dq, dk, dv = oat.attn_bwd(x["q"], x["k"], x["v"], lse, x["do"], heads=heads, **kw)
    tq, tk = grad_term_scales(x, o, lse, heads=heads, **kw)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dq_terms": tq, "dk_terms": tk}


def compare(got, ref, tol, heads=None, kv_heads=None):
    """Per-tensor and per-row max-norm relative errors within tol (rows: the
    head-dim vector of each query for O and dQ and of each key for dK and dV,
    each query's LSE); returns the per-tensor figures and prints the
    elementwise ones."""
    errs, elem = {}, {}
    for name in ("o", "lse", "dq", "dk", "dv"):
        g, r = got[name], ref[name]
        floor = ref.get(name + "_terms")
        if heads is not None:
            if name == "dq":
                floor = np.stack([floor[bb, :, hh] for bb, hh in heads])
            elif name == "dk":
                floor = np.stack([floor[bb, :, kk] for bb, kk in kv_heads])
            if name == "lse":
                g = np.stack([g[bb, hh] for bb, hh in heads]); r = np.stack([r[bb, hh] for bb, hh in heads])
            elif name in ("o", "dq"):
                g = np.stack([g[bb, :, hh] for bb, hh in heads]); r = np.stack([r[bb, :, hh] for bb, hh in heads])
            else:
                g = np.stack([g[bb, :, kk] for bb, kk in kv_heads]); r = np.stack([r[bb, :, kk] for bb, kk in kv_heads])
        errs[name] = assert_close(name, g, r, tol, row_len=1 if name == "lse" else g.shape[-1], row_floor=floor)
        elem[name] = f"{elementwise_err(g, r):.2e}"
    print("elementwise (reported, not gated):", elem)
    return errs


def test_tiny_fp32_workload():
    device = need_gpu()
    a = gen.WORKLOADS["tiny-fp32"].attn
    announce(f"attention tiny-fp32 {a}")
    x = gen.attn_inputs(a)
    errs = compare(run_gpu(a, x, device), run_oracle(a, x), TOL_FP32)
    print(errs)


SMALL = [
    # b, s, hq, hkv, d, causal, p
    (1, 1, 1, 1, 64, True, 0.1),
    (1, 37, 2, 2, 32, False, 0.1),
    (2, 130, 2, 1, 64, True, 0.1),
    (1, 257, 3, 3, 96, True, 0.1),
    (1, 200, 2, 2, 96, False, 0.0),
    (1, 384, 4, 2, 128, True, 0.1),
    (1, 300, 2, 2, 128, False, 0.3),
    (1, 261, 2, 2, 160, True, 0.1),
    (2, 150, 4, 2, 160, False, 0.1),   # producer/consumer dK/dV: grouped, non-causal, dropout
    (1, 190, 4, 1, 128, False, 0.2),   # two-group forward / dQ, producer/consumer dK/dV: 4:1, non-causal
    (2, 128, 8, 1, 128, True, 0.0),
    (1, 333, 2, 2, 192, True, 0.1),
    (2, 200, 4, 2, 192, False, 0.0),
    (1, 300, 2, 2, 256, True, 0.1),
    (2, 130, 4, 2, 256, False, 0.0),
]


def _swept_shapes(n=20, seed=2026):
    """Seeded draws over the supported space: every head dim, grouped-query
    ratios, lengths from 1 to 320 (tails of every tile size), causal or not,
    with and without dropout."""
    r = np.random.RandomState(seed)
    out = []
    for _ in range(n):
        hkv = int(r.choice([1, 2, 3]))
        hq = hkv * int(r.choice([1, 2, 4]))
        out.append((int(r.randint(1, 3)), int(r.randint(1, 321)), hq, hkv, int(r.choice([32, 64, 96, 128, 160, 192, 256])),
                    bool(r.randint(2)), float(r.choice([0.0, 0.1, 0.25]))))
    return out


@pytest.mark.parametrize("b,s,hq,hkv,d,causal,p", SMALL + _swept_shapes())
def test_bf16_small_shapes(b, s, hq, hkv, d, causal, p):
    device = need_gpu()
    a = gen.AttnShape(b=b, s=s, hq=hq, hkv=hkv, d=d, causal=causal, p_drop=p, seed=1234, head_offset=3)
    announce(f"attention bf16 {a}")
    x = gen.attn_inputs(a, seed_base=17)
    errs = compare(run_gpu(a, x, device), run_oracle(a, x), TOL_BF16)
    print(errs)


@pytest.mark.parametrize("b,s,hq,hkv,d,causal,p", [(1, 100, 4, 2, 128, True, 0.2), (2, 70, 2, 2, 160, False, 0.1),
                                                   (1, 64, 2, 1, 96, True, 0.0)])
def test_fp32_path_shapes(b, s, hq, hkv, d, causal, p):
    device = need_gpu()
    a = gen.AttnShape(b=b, s=s, hq=hq, hkv=hkv, d=d, causal=causal, p_drop=p, seed=7, dtype="fp32", in_scale=1.0)
    announce(f"attention fp32 {a}")
    x = gen.attn_inputs(a, seed_base=5)
    compare(run_gpu(a, x, device), run_oracle(a, x), TOL_FP32)


def test_mask_dump_bit_exact():
    device = need_gpu()
    b, s, hq, p, seed, off = 2, 67, 3, 0.1, 0xABCDEF0123, 5
    announce(f"attention mask dump b={b} s={s} hq={hq}")
    m = ops.attn_dropout_mask(b, s, hq, p_drop=p, seed=seed, head_offset=off, device=device).cpu().numpy()
    for bb in range(b):
        for hh in range(hq):
            ref = oph.attn_keep_mask(seed, p, bb, off + hh, s, s)
            np.testing.assert_array_equal(m[bb, hh].astype(bool), ref)


@pytest.mark.parametrize("causal", [True, False])
def test_forward_mask_black_box(causal):
    """V one-hot over a block of d keys makes O reveal P_d, so the kernel's
    forward mask is read from O != 0 and must equal the oracle's bit for bit."""
    device = need_gpu()
    b, s, hq, d, p, seed = 1, 192, 2, 64, 0.25, 99
    announce(f"forward mask probe causal={causal}")
    rng = np.random.default_rng(0)
    q = torch.tensor(rng.standard_normal((b, s, hq, d)) * 0.3, dtype=torch.bfloat16, device=device)
    k = torch.tensor(rng.standard_normal((b, s, hq, d)) * 0.3, dtype=torch.bfloat16, device=device)
    for j0 in range(0, s, d):
        v = torch.zeros((b, s, hq, d), dtype=torch.bfloat16, device=device)
        idx = torch.arange(d, device=device)
        v[:, j0 + idx, :, idx] = 1.0
        o, _ = ops.attn_core_fwd(q, k, v, causal=causal, p_drop=p, seed=seed)
        o = o.float().cpu().numpy()
        for hh in range(hq):
            ref = oph.attn_keep_mask(seed, p, 0, hh, s, s)[:, j0:j0 + d]
            vis = np.ones((s, d), bool) if not causal else (np.arange(s)[:, None] >= j0 + np.arange(d)[None, :])
            got = o[0, :, hh, :] != 0
            np.testing.assert_array_equal(got[vis], ref[vis])
            assert not got[~vis].any()


def test_backward_mask_black_box():
    """dO one-hot over a block of d queries makes dV reveal P_d^T: the mask the
    backward regenerates equals the oracle's (and so the forward's)."""
    device = need_gpu()
    b, s, hq, d, p, seed = 1, 128, 1, 64, 0.3, 5
    announce("backward mask probe")
    rng = np.random.default_rng(1)
    q = torch.tensor(rng.standard_normal((b, s, hq, d)) * 0.3, dtype=torch.bfloat16, device=device)
    k = torch.tensor(rng.standard_normal((b, s, hq, d)) * 0.3, dtype=torch.bfloat16, device=device)
    v = torch.tensor(rng.standard_normal((b, s, hq, d)), dtype=torch.bfloat16, device=device)
    o, lse = ops.attn_core_fwd(q, k, v, causal=False, p_drop=p, seed=seed)
    ref = oph.attn_keep_mask(seed, p, 0, 0, s, s)
    for i0 in range(0, s, d):
        do = torch.zeros_like(o)
        idx = torch.arange(d, device=device)
        do[:, i0 + idx, :, idx] = 1.0
        _, _, dv = ops.attn_core_bwd(q, k, v, o, lse, do, causal=False, p_drop=p, seed=seed)
        dvh = dv.float().cpu().numpy()[0, :, 0, :]          # [key j, c] = P_d[i0 + c, j]
        np.testing.assert_array_equal(dvh.T != 0, ref[i0:i0 + d, :])


def test_forward_and_backward_are_deterministic():
    device = need_gpu()
    a = gen.AttnShape(b=1, s=512, hq=4, hkv=4, d=128, causal=True, p_drop=0.1)
    announce("determinism")
    x = gen.attn_inputs(a)
    r1 = run_gpu(a, x, device)
    r2 = run_gpu(a, x, device)
    # no atomics anywhere: every output, gradients included, is reproducible bit for bit
    for n in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(r1[n], r2[n])


def test_gqa_backward_is_deterministic():
    device = need_gpu()
    a = gen.AttnShape(b=1, s=320, hq=8, hkv=2, d=128, causal=True, p_drop=0.1)
    announce("determinism gqa")
    x = gen.attn_inputs(a)
    r1 = run_gpu(a, x, device)
    r2 = run_gpu(a, x, device)
    for n in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(r1[n], r2[n])


def test_head_offset_split_invariance():
    """Two tensor-parallel ranks with heads [0,2) and [2,4) reproduce the 4-head run."""
    device = need_gpu()
    a = gen.AttnShape(b=2, s=200, hq=4, hkv=4, d=64, causal=True, p_drop=0.2, seed=3)
    announce("head split invariance")
    x = gen.attn_inputs(a)
    full = run_gpu(a, x, device)
    for lo in (0, 2):
        sub = {n: x[n][:, :, lo:lo + 2] for n in x}
        part = run_gpu(a.with_(hq=2, hkv=2, head_offset=lo), sub, device)
        np.testing.assert_array_equal(part["o"], full["o"][:, :, lo:lo + 2])
        np.testing.assert_array_equal(part["lse"], full["lse"][:, lo:lo + 2])
        for n in ("dq", "dk", "dv"):        # per-head work is independent of the split
            np.testing.assert_array_equal(part[n], full[n][:, :, lo:lo + 2])


def test_paired_grid_equals_unpaired():
    """At d = 128 a causal dK/dV grid with enough (batch, head) pairs runs two
    key blocks per workgroup (blocks t and n-1-t); each block's arithmetic is
    unchanged, so the heads it shares with a smaller, unpaired grid come out
    bit for bit the same (forward and dQ included)."""
    device = need_gpu()
    a = gen.AttnShape(b=1, s=2048, hq=32, hkv=32, d=128, causal=True, p_drop=0.1, seed=11)
    announce("paired grid (32 heads) against unpaired (24 heads)")
    x = gen.attn_inputs(a)
    full = run_gpu(a, x, device)                  # 32 x 8 pairs: paired
    sub = {n: x[n][:, :, :24] for n in x}
    part = run_gpu(a.with_(hq=24, hkv=24), sub, device)   # 24 x 8 < 256: not paired, not split
    np.testing.assert_array_equal(part["o"], full["o"][:, :, :24])
    np.testing.assert_array_equal(part["lse"], full["lse"][:, :24])
    for n in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(part[n], full[n][:, :, :24])


def test_no_s_by_s_allocation():
    device = need_gpu()
    a = gen.AttnShape(b=1, s=4096, hq=8, hkv=1, d=128, causal=True, p_drop=0.0)
    announce("peak memory")
    x = gen.attn_inputs(a)
    q, k, v, do = (dev(x[n], "bf16", device) for n in ("q", "k", "v", "do"))
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(device)
    base = torch.cuda.memory_allocated(device)
    o, lse = ops.attn_core_fwd(q, k, v, causal=True)
    dq, dk, dv = ops.attn_core_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    growth = torch.cuda.max_memory_allocated(device) - base
    assert growth < a.b * a.hq * a.s * a.s, f"peak growth {growth} bytes reaches the s^2 scale"


@pytest.mark.parametrize("name", ["gpt22b-t8", "gpt175b-t8", "gpt530b-t8", "llama3-70b-t8"])
def test_full_size_workload_sampled_heads(name):
    """Full-size inputs in the configuration the bench times; the oracle checks
    every head of the first and last batch element (b > 1), four heads
    (b = 1), or every q-head of kv-head 0 (grouped-query attention)."""
    device = need_gpu()
    a = gen.WORKLOADS[name].attn
    announce(f"full-size {name}")
    x = gen.attn_inputs(a)
    got = run_gpu(a, x, device)
    grp = a.hq // a.hkv
    if grp == 1 and a.b > 1:
        # every head of the first and the last batch element
        heads = [(bb, hh) for bb in (0, a.b - 1) for hh in range(a.hq)]
        kv = heads
    elif grp == 1:
        heads = [(0, hh) for hh in (0, a.hq // 3, 2 * a.hq // 3, a.hq - 1)]
        kv = heads
    else:
        heads = [(0, h) for h in range(grp)]          # every q-head of kv-head 0
        kv = [(0, 0)]
    ref = run_oracle(a, x, heads=heads)
    print(name, compare(got, ref, TOL_BF16, heads=heads, kv_heads=kv))


def test_strided_views_of_a_fused_qkv_buffer():
    """Q, K, V as views into one [b, s, 3, h, d] buffer (the layout a fused QKV
    GEMM writes): the results equal those of contiguous copies bit for bit,
    and dQ, dK, dV come back with the views' strides."""
    device = need_gpu()
    a = gen.AttnShape(b=2, s=190, hq=4, hkv=4, d=96, causal=True, p_drop=0.1, seed=11)
    announce("strided qkv views")
    x = gen.attn_inputs(a)
    contiguous = run_gpu(a, x, device)
    qkv = torch.empty((a.b, a.s, 3, a.hq, a.d), dtype=torch.bfloat16, device=device)
    for i, n in enumerate(("q", "k", "v")):
        qkv[:, :, i] = dev(x[n], "bf16", device)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    assert not q.is_contiguous()
    do = dev(x["do"], "bf16", device)
    kw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed, head_offset=a.head_offset)
    o, lse = ops.attn_core_fwd(q, k, v, **kw)
    dq, dk, dv = ops.attn_core_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    assert dq.stride() == q.stride() and dk.stride() == k.stride() and dv.stride() == v.stride()
    for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_array_equal(host(t), contiguous[n])


@pytest.mark.parametrize("b,s", [(0, 64), (2, 0)])
def test_empty_batch_or_sequence(b, s):
    """Zero-sized inputs are valid: the calls succeed, launch nothing and
    return empty outputs."""
    device = need_gpu()
    announce(f"empty attention b={b} s={s}")
    q = torch.empty((b, s, 2, 64), dtype=torch.bfloat16, device=device)
    o, lse = ops.attn_core_fwd(q, q, q, causal=True, p_drop=0.1)
    dq, dk, dv = ops.attn_core_bwd(q, q, q, o, lse, torch.empty_like(o), causal=True, p_drop=0.1)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (b, 2, s) and dq.shape == q.shape


def test_forward_split_grid_and_unsplit_agree_with_the_oracle():
    """A small causal grid at d = 128 can split its longest query tiles over
    two workgroups (with a workspace) or not (without one): both match the
    oracle, and the merged LSE equals the unsplit one to the rounding of the
    row sums, which add the bf16-rounded probabilities (each within 2^-9 of
    its value; the two launches round against different running maxima, so
    their log-sums can differ by up to 2^-8)."""
    device = need_gpu()
    a = gen.AttnShape(b=1, s=384, hq=4, hkv=2, d=128, causal=True, p_drop=0.1, seed=21)
    announce("forward split vs unsplit")
    x = gen.attn_inputs(a)
    q, k, v = (dev(x[n], "bf16", device) for n in ("q", "k", "v"))
    kw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed, head_offset=a.head_offset)
    o1 = torch.empty_like(q)
    l1 = torch.empty((a.b, a.hq, a.s), dtype=torch.float32, device=device)
    desc = ops.attn_desc(q, k, v, o1, head_offset=0, **{n: kw[n] for n in ("causal", "scale", "p_drop", "seed")})
    assert ops.attn_fwd_workspace_bytes(desc) > 0
    ops.prepare_attn_fwd(q, k, v, o1, l1, workspace=None, **kw)()          # unsplit
    o2, l2 = ops.attn_core_fwd(q, k, v, **kw)                              # split (workspace allocated)
    torch.cuda.synchronize()
    o_ref, lse_ref = oat.attn_fwd(x["q"], x["k"], x["v"], **kw)
    assert_close("o unsplit", host(o1), o_ref, TOL_BF16)
    assert_close("o split", host(o2), o_ref, TOL_BF16)
    np.testing.assert_allclose(host(l2), host(l1), rtol=0, atol=2.0**-8)


PADDED = [
    # b, s, hq, hkv, d, causal, p, valid lengths
    (4, 200, 2, 2, 64, True, 0.1, [200, 0, 77, 129]),
    (3, 300, 4, 2, 128, True, 0.1, [1, 300, 150]),
    (2, 257, 3, 3, 96, False, 0.2, [256, 33]),
    (2, 384, 2, 1, 160, True, 0.0, [383, 64]),
    (2, 300, 2, 2, 192, True, 0.1, [300, 111]),
    (2, 260, 2, 1, 256, True, 0.1, [260, 99]),
    (4, 2048, 8, 8, 96, True, 0.1, [2048, 1500, 700, 31]),
    # 32 (batch, head) pairs of 16 key blocks: the d = 128 dK/dV grid runs paired
    (2, 2048, 16, 16, 128, True, 0.1, [2048, 1337]),
]


@pytest.mark.parametrize("b,s,hq,hkv,d,causal,p,lens", PADDED)
def test_padded_batch(b, s, hq, hkv, d, causal, p, lens):
    """Per-element valid lengths: O, LSE and the gradients match the oracle's
    padded-batch definition; padded positions are exactly O = 0, LSE = -inf,
    dQ = dK = dV = 0."""
    device = need_gpu()
    a = gen.AttnShape(b=b, s=s, hq=hq, hkv=hkv, d=d, causal=causal, p_drop=p, seed=99, head_offset=1)
    announce(f"padded batch {a} lens={lens}")
    x = gen.attn_inputs(a, seed_base=31)
    q, k, v, do = (dev(x[n], "bf16", device) for n in ("q", "k", "v", "do"))
    sl = torch.tensor(lens, dtype=torch.int32, device=device)
    kw = dict(causal=causal, scale=a.scale, p_drop=p, seed=a.seed, head_offset=a.head_offset)
    o, lse = ops.attn_core_fwd(q, k, v, seqlens=sl, **kw)
    dq, dk, dv = ops.attn_core_bwd(q, k, v, o, lse, do, seqlens=sl, **kw)
    torch.cuda.synchronize()
    heads = None if s <= 512 else [(0, 0), (1, 3), (2, 5), (3, 7)][:b]
    o_r, lse_r = oat.attn_fwd(x["q"], x["k"], x["v"], heads=heads, seqlens=lens, **kw)
    dq_r, dk_r, dv_r = oat.attn_bwd(x["q"], x["k"], x["v"], lse_r, x["do"], heads=heads, seqlens=lens, **kw)
    tq, tk = grad_term_scales(x, o_r, lse_r, heads=heads, seqlens=lens, **kw)
    got = {"o": host(o), "lse": host(lse), "dq": host(dq), "dk": host(dk), "dv": host(dv)}
    pairs = heads or [(bb, hh) for bb in range(b) for hh in range(hq)]
    grp = hq // hkv
    for bb, hh in pairs:
        L = lens[bb]
        g = hh // grp
        assert np.all(np.isneginf(got["lse"][bb, hh, L:]))
        assert not got["o"][bb, L:, hh].any() and not got["dq"][bb, L:, hh].any()
        assert not got["dk"][bb, L:, g].any() and not got["dv"][bb, L:, g].any()
        if L == 0:
            continue
        assert_close("lse", got["lse"][bb, hh, :L], lse_r[bb, hh, :L], TOL_BF16, row_len=1)
        assert_close("o", got["o"][bb, :L, hh], o_r[bb, :L, hh], TOL_BF16, row_len=d)
        assert_close("dq", got["dq"][bb, :L, hh], dq_r[bb, :L, hh], TOL_BF16, row_len=d,
                     row_floor=tq[bb, :L, hh])
        if heads is None or grp == 1:
            assert_close("dk", got["dk"][bb, :L, g], dk_r[bb, :L, g], TOL_BF16, row_len=d,
                         row_floor=tk[bb, :L, g])
            assert_close("dv", got["dv"][bb, :L, g], dv_r[bb, :L, g], TOL_BF16, row_len=d)


def test_full_lengths_equal_no_lengths():
    """seqlens all equal to s gives the unpadded results bit for bit."""
    device = need_gpu()
    a = gen.AttnShape(b=2, s=320, hq=4, hkv=2, d=128, causal=True, p_drop=0.1, seed=5)
    announce("full lengths")
    x = gen.attn_inputs(a)
    ref = run_gpu(a, x, device)
    q, k, v, do = (dev(x[n], "bf16", device) for n in ("q", "k", "v", "do"))
    sl = torch.full((a.b,), a.s, dtype=torch.int32, device=device)
    kw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed, head_offset=a.head_offset)
    o, lse = ops.attn_core_fwd(q, k, v, seqlens=sl, **kw)
    dq, dk, dv = ops.attn_core_bwd(q, k, v, o, lse, do, seqlens=sl, **kw)
    torch.cuda.synchronize()
    for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_array_equal(host(t), ref[n])
