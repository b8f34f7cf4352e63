"""The seeded input generator: bf16 rounding and workload shapes."""
import numpy as np
import torch

from selective_recompute_attention_attn_amd import gen


def test_round_to_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0, 65504.0],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(gen.round_to_bf16(x), want)


def test_inputs_are_seeded_and_shaped():
    w = gen.WORKLOADS["tiny-fp32"]
    a1 = gen.attn_inputs(w.attn)
    a2 = gen.attn_inputs(w.attn)
    for k in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(a1[k], a2[k])
    assert a1["q"].shape == (1, 128, 2, 32) and a1["k"].shape == (1, 128, 2, 32)
    n = gen.norm_inputs(w.norm)
    assert n["resid"].shape == (128, 1, 64) and n["gamma"].shape == (64,)


def test_bf16_inputs_are_representable():
    a = gen.AttnShape(b=1, s=64, hq=2, hkv=1, d=32, causal=True, p_drop=0.1)
    x = gen.attn_inputs(a)["q"]
    np.testing.assert_array_equal(gen.round_to_bf16(x), x)
    assert np.abs(x).max() < 4.0   # N(0,1) * 0.5


def test_workload_table():
    w = gen.WORKLOADS
    assert w["gpt22b-t8"].attn.d * 64 == 6144 and w["gpt22b-t8"].norm.rows == 1024
    assert w["gpt175b-t8"].attn.hq * 8 * w["gpt175b-t8"].attn.d == 12288
    assert w["gpt530b-t8"].attn.hq * 8 * w["gpt530b-t8"].attn.d == 20480
    l = w["llama3-70b-t8"].attn
    assert (l.hq, l.hkv, l.s, l.p_drop) == (8, 1, 8192, 0.0)
