"""The library's recompute-policy calls (host only, no GPU) against the oracle's
exact brute-force planner: layer counts bit-exact, bytes and extra compute to
double rounding."""
import random
from fractions import Fraction

import pytest

from oracle import ledger as lg
from selective_recompute_attention_attn_amd import ops


@pytest.fixture(scope="module")
def L():
    return ops.lib()


def _shapes():
    rng = random.Random(7)
    out = [dict(s=8192, b=1, h=8192, a=64, layers=80, n_params=70 * 10**9, t=1, sequence_parallel=False, causal=True),
           dict(s=2048, b=4, h=6144, a=64, layers=48, n_params=22 * 10**9, t=8, sequence_parallel=True, causal=True),
           dict(s=2048, b=1, h=20480, a=128, layers=105, n_params=530 * 10**9, t=8, sequence_parallel=False, causal=True)]
    for _ in range(12):
        a = rng.choice((8, 16, 32, 64))
        out.append(dict(s=rng.choice((128, 512, 1000, 4096)), b=rng.randint(1, 6), h=a * rng.choice((64, 96, 128)),
                        a=a, layers=rng.randint(1, 40), n_params=rng.choice((0, 10**8, 7 * 10**9)),
                        t=rng.choice((1, 2, 3, 8)), sequence_parallel=rng.random() < 0.5, causal=rng.random() < 0.5))
    return out


@pytest.mark.parametrize("kw", _shapes())
def test_policy_bytes_and_cost_match_oracle(kw):
    for pol in lg.POLICIES:
        nb, ex = ops.activation_bytes(pol, **kw)
        want_b = lg.layer_bytes_exact(kw["s"], kw["b"], kw["h"], kw["a"], kw["t"], kw["sequence_parallel"], pol)
        ns = kw["layers"] if pol == "selective" else 0
        nf = kw["layers"] if pol == "full" else 0
        want_x = lg.extra_compute_exact(kw["s"], kw["h"], kw["layers"], kw["n_params"], kw["causal"], ns, nf)
        assert nb == pytest.approx(float(want_b), rel=1e-15)
        assert ex == pytest.approx(float(want_x), rel=1e-15, abs=0)


@pytest.mark.parametrize("kw", _shapes())
def test_plan_matches_oracle_brute_force(kw):
    mem = {p: lg.layer_bytes_exact(kw["s"], kw["b"], kw["h"], kw["a"], kw["t"], kw["sequence_parallel"], p)
           for p in lg.POLICIES}
    n = kw["layers"]
    lo, hi = n * mem["full"], n * mem["none"]
    rng = random.Random(kw["s"] * 31 + n)
    budgets = [float(lo), float(hi), float(hi) * 2, float(lo + (hi - lo) / 3)]
    budgets += [float(lo + (hi - lo) * Fraction(rng.random())) for _ in range(10)]
    for budget in budgets:
        want = lg.plan_recompute(budget, **kw)
        if want is None:
            with pytest.raises(ops.SratError, match="UNSUPPORTED"):
                ops.plan_recompute(budget, **kw)
            continue
        got = ops.plan_recompute(budget, **kw)
        assert (got["none"], got["selective"], got["full"]) == want[:3], budget
        assert got["activation_bytes"] == pytest.approx(float(want[3]), rel=1e-15)
        assert got["extra_compute"] == pytest.approx(float(want[4]), rel=1e-15, abs=0)


def test_budget_below_full_is_refused_and_plan_zeroed(L):
    kw = dict(s=1024, b=1, h=1024, a=8, layers=4)
    full = 4 * float(lg.layer_bytes_exact(1024, 1, 1024, 8, 1, False, "full"))
    assert ops.plan_recompute(full, **kw)["full"] == 4
    plan = ops.RecomputePlan(1, 2, 3, 4.0, 5.0)
    d = ops.layer_desc(**kw)
    import ctypes
    assert L.srat_plan_recompute(ctypes.byref(d), full - 1, ctypes.byref(plan)) == -2
    assert (plan.layers_none, plan.layers_selective, plan.layers_full, plan.activation_bytes) == (0, 0, 0, 0.0)


@pytest.mark.parametrize("bad", [dict(s=0), dict(h=-1), dict(layers=0), dict(t=0), dict(n_params=-5),
                                 dict(a=0), dict(s=1 << 41), dict(layers=1 << 20), dict(t=1 << 20),
                                 dict(s=1 << 30, b=1 << 30, h=1)])
def test_invalid_layer_desc(bad):
    kw = dict(s=1024, b=1, h=1024, a=8, layers=4)
    kw.update(bad)
    with pytest.raises(ops.SratError, match="INVALID"):
        ops.activation_bytes("none", **kw)
    with pytest.raises(ops.SratError, match="INVALID"):
        ops.plan_recompute(1e12, **kw)


def test_unknown_policy_and_null_pointers(L):
    import ctypes
    d = ops.layer_desc(s=128, b=1, h=64, a=2, layers=2)
    assert L.srat_activation_bytes(ctypes.byref(d), 3, None, None) == -1
    assert L.srat_activation_bytes(None, 0, None, None) == -1
    assert L.srat_activation_bytes(ctypes.byref(d), 0, None, None) == 0
    assert L.srat_plan_recompute(ctypes.byref(d), 1e9, None) == -1


@pytest.mark.parametrize("budget", [-1.0, float("nan")])
def test_negative_or_nan_budget_is_invalid(budget):
    with pytest.raises(ops.SratError, match="INVALID"):
        ops.plan_recompute(budget, s=128, b=1, h=64, a=2, layers=2)
