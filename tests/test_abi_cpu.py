"""The C-ABI library on the CPU: it loads, exports what include/srat.h declares,
validates arguments before any HIP call, and its Philox agrees with the oracle."""
import ctypes
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox as ph
from selective_recompute_attention_attn_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "srat.h")
CSRC = os.path.join(ROOT, "selective_recompute_attention_attn_amd", "csrc")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        pytest.fail("libsrat.so is not built (run __graft_entry__.build())")
    return ops.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(srat_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(ops.EXPORTS)
    assert L.srat_version() == 2


def _desc(**kw):
    base = dict(dtype=ops.SRAT_BF16, causal=1, b=1, s=256, hq=4, hkv=4, d=64,
                q_stride=(256 * 4 * 64, 4 * 64, 64), k_stride=(256 * 4 * 64, 4 * 64, 64),
                v_stride=(256 * 4 * 64, 4 * 64, 64), o_stride=(256 * 4 * 64, 4 * 64, 64),
                scale=0.125, p_drop=0.1, seed=0, head_offset=0)
    base.update(kw)
    for k in ("q_stride", "k_stride", "v_stride", "o_stride"):
        base[k] = (ctypes.c_int64 * 3)(*base[k])
    return ops.AttnDesc(**base)


def _err(L, rc):
    return rc, L.srat_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(d=48), -2), (dict(d=320), -2), (dict(d=192, dtype=ops.SRAT_F32), -2), (dict(d=256, dtype=ops.SRAT_F32), -2), (dict(p_drop=1.0), -1), (dict(p_drop=-0.1), -1),
    (dict(hq=4, hkv=3), -1), (dict(dtype=7), -1), (dict(causal=2), -1), (dict(s=-1), -1),
    (dict(q_stride=(256 * 4 * 64, 4 * 64, 60)), -1), (dict(k_stride=(0, 3, 64)), -1),
    (dict(head_offset=-1), -1), (dict(scale=float("nan")), -1), (dict(scale=float("inf")), -1),
    (dict(scale=-0.1), -1), (dict(p_drop=1.0 - 2.0**-18), -1), (dict(p_drop=0.999995), -1)])
def test_attention_validation_before_any_hip_call(L, kw, code):
    d = _desc(**kw)
    n = ctypes.c_size_t(0)
    rc, msg = _err(L, L.srat_attn_core_bwd_workspace(ctypes.byref(d), ctypes.byref(n)))
    assert rc == code and msg
    # forward with NULL tensors: the descriptor error comes first
    rc, msg = _err(L, L.srat_attn_core_fwd(ctypes.byref(d), None, None, None, None, None, None))
    assert rc == code and msg


def test_null_descriptor_and_null_pointers(L):
    assert L.srat_attn_core_fwd(None, None, None, None, None, None, None) == -1
    d = _desc()
    rc, msg = _err(L, L.srat_attn_core_fwd(ctypes.byref(d), None, None, None, None, None, None))
    assert rc == -1 and "NULL" in msg
    odd = ctypes.c_void_p(0x1002)
    rc, msg = _err(L, L.srat_attn_core_fwd(ctypes.byref(d), odd, odd, odd, odd, odd, None))
    assert rc == -1
    rc, msg = _err(L, L.srat_attn_core_bwd(ctypes.byref(d), *([ctypes.c_void_p(0x1000)] * 9),
                                           ctypes.c_void_p(0x1000), 16, None))
    assert rc == -3 and "workspace" in msg


def test_noalloc_backward_refuses_oversized_shapes_before_any_hip_call(L):
    """The allocation-free backward takes its workspace from a fixed scratch
    array: a shape needing more is refused with SRAT_ERR_UNSUPPORTED, and bad
    descriptors and pointers are refused as by srat_attn_core_bwd, all before
    any HIP call (so on a machine without a GPU)."""
    limit = 128 << 20
    fake = [ctypes.c_void_p(0x10000)] * 9
    hq, d = 8, 128
    for s, ok in ((8192, True), (32768, False)):
        qs, ks = (s * hq * d, hq * d, d), (s * d, d, d)
        desc = _desc(s=s, hq=hq, hkv=1, d=d, q_stride=qs, o_stride=qs, k_stride=ks, v_stride=ks)
        n = ctypes.c_size_t(0)
        assert L.srat_attn_core_bwd_workspace(ctypes.byref(desc), ctypes.byref(n)) == 0
        assert (n.value <= limit) == ok
        if not ok:
            rc, msg = _err(L, L.srat_attn_core_bwd_noalloc(ctypes.byref(desc), *fake, None))
            assert rc == -2 and "no-allocation" in msg and str(limit) in msg
    rc, msg = _err(L, L.srat_attn_core_bwd_noalloc(ctypes.byref(_desc()), *([None] * 9), None))
    assert rc == -1 and "NULL" in msg
    rc, _ = _err(L, L.srat_attn_core_bwd_noalloc(ctypes.byref(_desc(d=48)), *fake, None))
    assert rc == -2


def test_workspace_is_linear_in_s_never_quadratic(L):
    """The backward workspace holds per-row data only: D (4 bytes per query
    row) plus, for grouped-query heads or split grids, at most two fp32 slots
    each of dK, dV and dQ partials (24 d bytes per row) -- never O(s^2)."""
    hq, d = 8, 128
    for s in (1024, 2048, 4096, 8192, 32768):
        qs, ks = (s * hq * d, hq * d, d), (s * d, d, d)
        desc = _desc(s=s, hq=hq, hkv=1, d=d, q_stride=qs, o_stride=qs, k_stride=ks, v_stride=ks)
        n = ctypes.c_size_t(0)
        assert L.srat_attn_core_bwd_workspace(ctypes.byref(desc), ctypes.byref(n)) == 0
        rows = s * hq
        assert rows * 4 <= n.value <= rows * (4 + 24 * d) + 4 * 256
        if s >= 8192:
            assert n.value < 2 * hq * s * s      # below one bf16 s x s matrix per q-head


def _ndesc(**kw):
    base = dict(dtype=ops.SRAT_BF16, norm=ops.SRAT_LAYERNORM, s_local=256, b=4, h=6144, seq_offset=0,
                eps=1e-5, p_drop=0.1, seed=0, site=1)
    base.update(kw)
    return ops.NormDesc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(h=100), -2), (dict(h=65536), -2), (dict(norm=3), -1), (dict(p_drop=1.0), -1),
    (dict(site=200), -1), (dict(b=0), -1), (dict(eps=-1.0), -1), (dict(seq_offset=-5), -1),
    (dict(p_drop=1.0 - 2.0**-18), -1),
    # the backward's grid (column workgroups + one per row) must fit 2^32 work-items
    (dict(h=256, s_local=1 << 26, b=1), -2), (dict(h=6144, s_local=1 << 23, b=2), -2)])
def test_norm_validation_before_any_hip_call(L, kw, code):
    d = _ndesc(**kw)
    n = ctypes.c_size_t(0)
    rc, msg = _err(L, L.srat_sp_norm_bwd_workspace(ctypes.byref(d), ctypes.byref(n)))
    assert rc == code and msg


def test_norm_alias_rule_and_workspace(L):
    d = _ndesc()
    n = ctypes.c_size_t(0)
    assert L.srat_sp_norm_bwd_workspace(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == 0          # dgamma / dbeta are summed without scratch memory
    p = ctypes.c_void_p(0x10000)
    rc, msg = _err(L, L.srat_sp_norm_bwd(ctypes.byref(d), p, p, p, p, p, p, p, p, p, p, p, n.value, None))
    assert rc == -1 and "alias" in msg


def test_trace_read_empty(L):
    assert L.srat_trace_enable(0) == 0
    assert L.srat_trace_read(None, 0, 1) >= 0


@pytest.fixture(scope="module")
def philox_hpp():
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    out = os.path.join(tempfile.mkdtemp(prefix="srat_hpp_"), "drv")
    subprocess.run([cxx, "-O2", f"-I{CSRC}", os.path.join(ROOT, "tests", "support", "philox_hpp_driver.cpp"),
                    "-o", out], check=True, capture_output=True)
    return out


def test_library_philox_equals_oracle(philox_hpp):
    rng = np.random.default_rng(3)
    rows = []
    for _ in range(2000):
        seed = int(rng.integers(0, 2**63)) * 2 + 1
        c = [int(x) for x in rng.integers(0, 2**32, size=4, dtype=np.uint64)]
        t = int(rng.choice([0, 1, 6554, 32768, 65535]))
        rows.append((seed, *c, t))
    inp = "".join(" ".join(map(str, r)) + "\n" for r in rows)
    res = subprocess.run([philox_hpp], input=inp, capture_output=True, text=True, check=True)
    for r, ln in zip(rows, res.stdout.strip().splitlines()):
        seed, c0, c1, c2, c3, t = r
        words = ph.philox4x32_10(c0, c1, c2, c3, seed & 0xFFFFFFFF, seed >> 32)
        parts = ln.split()
        assert [int(x, 16) for x in parts[:4]] == [int(w) for w in words]
        bits = 0
        for e in range(8):
            u = (int(words[e >> 1]) >> (16 * (e & 1))) & 0xFFFF
            bits |= int(u >= t) << e
        assert int(parts[4], 16) == bits
        assert [int(x, 16) for x in parts[5:9]] == [int(w) for w in words]   # row-hoisted form
        assert [int(x, 16) for x in parts[9:13]] == [int(w) for w in words]  # column-hoisted form


def test_threshold_rule_matches_oracle():
    # the host code computes T from the float probability in double precision
    for p in (0.0, 0.1, 0.25, 0.3333, 0.9999, 1.0 - 2.0**-16, 1.0 - 2.0**-17 - 2.0**-24):
        t = int(float(np.float32(p)) * 65536.0 + 0.5)
        assert t == ph.drop_threshold(p) and t <= 0xFFFF


@pytest.mark.parametrize("p", [1.0 - 2.0**-17, 1.0 - 2.0**-18, 0.999995, float(np.nextafter(np.float32(1), 0))])
def test_threshold_65536_refused_on_both_sides(L, p):
    """A p whose 16-bit threshold rounds to 65536 is refused by the oracle and
    by every entry point (attention and norm descriptors) before any HIP call:
    the kernels compare 16-bit halves against T and cannot express it."""
    assert int(float(np.float32(p)) * 65536.0 + 0.5) == 65536
    with pytest.raises(ValueError):
        ph.drop_threshold(p)
    n = ctypes.c_size_t(0)
    d = _desc(p_drop=p)
    rc, msg = _err(L, L.srat_attn_core_bwd_workspace(ctypes.byref(d), ctypes.byref(n)))
    assert rc == -1 and "65536" in msg
    nd = _ndesc(p_drop=p)
    rc, msg = _err(L, L.srat_sp_norm_bwd_workspace(ctypes.byref(nd), ctypes.byref(n)))
    assert rc == -1 and "65536" in msg


def test_scale_zero_means_the_default(L):
    """scale = 0 asks the library for 1/sqrt(d): the descriptor is valid and
    the binding passes 0 when no scale is given (the binding computes no part
    of the method)."""
    n = ctypes.c_size_t(0)
    d = _desc(scale=0.0)
    assert L.srat_attn_core_bwd_workspace(ctypes.byref(d), ctypes.byref(n)) == 0
    import torch
    z = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16)
    assert ops.attn_desc(z, z, z, z, causal=True, scale=None, p_drop=0.0, seed=0, head_offset=0).scale == 0.0
    assert ops.attn_desc(z, z, z, z, causal=True, scale=0.25, p_drop=0.0, seed=0, head_offset=0).scale == 0.25


def test_norm_row_limit_boundary(L):
    """The largest row count the backward grid holds is accepted, one more is not."""
    n = ctypes.c_size_t(0)
    for h in (256, 6144, 32768):
        groups = (h + 7) // 8
        blk = 64
        while blk < 1024 and (groups + blk - 1) // blk > 3:
            blk *= 2
        cols = 8 * (((h + 31) // 32 + 7) // 8)
        limit = min((2**32 - 1) // blk, 2**31 - 1) - cols
        ok = _ndesc(h=h, s_local=limit, b=1)
        assert L.srat_sp_norm_bwd_workspace(ctypes.byref(ok), ctypes.byref(n)) == 0, (h, L.srat_last_error())
        bad = _ndesc(h=h, s_local=limit + 1, b=1)
        assert _err(L, L.srat_sp_norm_bwd_workspace(ctypes.byref(bad), ctypes.byref(n)))[0] == -2


def test_seqlens_only_on_the_bf16_path(L):
    """Per-element lengths are a bf16-path feature: the fp32 path refuses them
    and a misaligned pointer is invalid, both before any HIP call."""
    n = ctypes.c_size_t(0)
    d = _desc(dtype=ops.SRAT_F32, seqlens=0x1000)
    assert _err(L, L.srat_attn_core_bwd_workspace(ctypes.byref(d), ctypes.byref(n)))[0] == -2
    d = _desc(seqlens=0x1002)
    assert _err(L, L.srat_attn_core_bwd_workspace(ctypes.byref(d), ctypes.byref(n)))[0] == -1
    d = _desc(seqlens=0x1000)
    assert L.srat_attn_core_bwd_workspace(ctypes.byref(d), ctypes.byref(n)) == 0


def test_plain_c_caller_against_the_oracle():
    """include/srat.h is usable from C alone: a C program built with the host
    compiler and linked against libsrat.so gets the workspace size, the
    validation error and the recompute plans the oracle computes."""
    from fractions import Fraction
    from oracle import ledger as lg
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    ops.lib()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "selective_recompute_attention_attn_amd")
    out = os.path.join(tempfile.mkdtemp(prefix="srat_c_"), "c_abi_example")
    subprocess.run([cc, "-std=c99", "-O1", "-I", os.path.join(root, "include"),
                    os.path.join(root, "tests", "support", "c_abi_example.c"), "-o", out,
                    "-L", pkg, "-lsrat", f"-Wl,-rpath,{pkg}"], check=True)
    lines = subprocess.run([out], check=True, capture_output=True, text=True).stdout.splitlines()
    got = {ln.split()[0] + (" " + ln.split()[1] if ln.startswith(("policy", "plan")) else ""): ln for ln in lines}
    assert got["version"] == "version 2"
    assert got["bwd_workspace"].startswith("bwd_workspace rc 0 ")
    assert "rc -2" in got["bad_head_dim"] and "head dim 48" in got["bad_head_dim"]
    kw = dict(s=8192, b=1, h=8192, a=64, layers=80, n_params=70 * 10**9, causal=True)
    for pol in lg.POLICIES:
        f = got[f"policy {pol}"].split()
        want_b = lg.layer_bytes_exact(8192, 1, 8192, 64, 1, False, pol)
        n = 80
        want_x = lg.extra_compute_exact(8192, 8192, n, 70 * 10**9, True, n if pol == "selective" else 0,
                                        n if pol == "full" else 0)
        assert f[3] == "0" and float(f[5]) == pytest.approx(float(want_b), rel=1e-15)
        assert float(f[7]) == pytest.approx(float(want_x), rel=1e-15, abs=0)
    for ln in lines:
        if not ln.startswith("plan "):
            continue
        f = ln.split()
        want = lg.plan_recompute(Fraction(float(f[1])), **kw)
        assert f[3] == "0" and (int(f[5]), int(f[7]), int(f[9])) == want[:3]
        assert float(f[11]) == pytest.approx(float(want[3]), rel=1e-15)
    assert got["too_small"] == "too_small rc -2"
