"""Seeded synthetic inputs and workload shapes.

This module is shared by the HIP path's callers (tests, bench) and by the
oracle's tests.  It holds shapes and random draws only -- no step of the
attention core or of the norm region is computed here.

Workloads are one tensor-parallel rank's share (t = 8) of the GPT-style
models in "Reducing Activation Recomputation in Large Transformer Models"
(Korthikanti et al.), plus a Llama-3-70B-style long-sequence layer and a tiny
fp32 correctness case.  Layouts:

* attention: Q, O, dO as ``[b, s, hq, d]``; K, V as ``[b, s, hkv, d]``
* norm region: ``[s_local, b, h]`` rows (sequence-major, as in the page's
  ``[s, b, h]`` activations split along s).

Every tensor is drawn in fp32 from ``numpy.random.default_rng(seed_base + id)``
(ids: q 0, k 1, v 2, do 3, resid 4, y 5, du 6, dres 7, gamma 8, beta 9),
scaled, then rounded to the workload dtype (bf16: round-to-nearest-even).  The
returned arrays are float32 holding exactly the dtype's values, so the oracle
sees precisely what the device sees.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "resid": 4, "y": 5, "du": 6,
              "dres": 7, "gamma": 8, "beta": 9}


@dataclass(frozen=True)
class AttnShape:
    """One rank's attention-core problem."""
    b: int
    s: int
    hq: int
    hkv: int
    d: int
    causal: bool
    p_drop: float
    seed: int = 0            # dropout Philox key
    head_offset: int = 0     # global index of local q-head 0
    dtype: str = "bf16"      # "bf16" or "fp32"
    in_scale: float = 0.5    # Q, K, V, dO ~ N(0, 1) * in_scale

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "AttnShape":
        return replace(self, **kw)


@dataclass(frozen=True)
class NormShape:
    """One rank's sequence-parallel LayerNorm/RMSNorm + dropout + residual."""
    s_local: int
    b: int
    h: int
    norm: str                # "layernorm" or "rmsnorm"
    p_drop: float
    seed: int = 0
    site: int = 1            # which hidden dropout (1: after attention, 2: after MLP)
    seq_offset: int = 0      # global sequence index of local row 0
    eps: float = 1e-5
    dtype: str = "bf16"
    gamma: str = "ones"      # "ones" or "u0.9-1.1"
    beta: str = "zeros"      # "zeros" or "n0.02"

    @property
    def rows(self) -> int:
        return self.s_local * self.b

    def with_(self, **kw) -> "NormShape":
        return replace(self, **kw)


@dataclass(frozen=True)
class Workload:
    name: str
    attn: AttnShape
    norm: NormShape


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 single layer, non-causal; the oracle finishes in well under a second
    "tiny-fp32": Workload(
        "tiny-fp32",
        AttnShape(b=1, s=128, hq=2, hkv=2, d=32, causal=False, p_drop=0.1,
                  dtype="fp32", in_scale=1.0),
        NormShape(s_local=128, b=1, h=64, norm="layernorm", p_drop=0.1, dtype="fp32")),
    # 22B GPT (h=6144, a=64) at t=8: 8 heads of 96, b=4, s=2048
    "gpt22b-t8": Workload(
        "gpt22b-t8",
        AttnShape(b=4, s=2048, hq=8, hkv=8, d=96, causal=True, p_drop=0.1),
        NormShape(s_local=256, b=4, h=6144, norm="layernorm", p_drop=0.1)),
    # 175B GPT (h=12288, a=96) at t=8: 12 heads of 128
    "gpt175b-t8": Workload(
        "gpt175b-t8",
        AttnShape(b=1, s=2048, hq=12, hkv=12, d=128, causal=True, p_drop=0.1),
        NormShape(s_local=256, b=1, h=12288, norm="layernorm", p_drop=0.1)),
    # 530B GPT (h=20480, a=128) at t=8: 16 heads of 160
    "gpt530b-t8": Workload(
        "gpt530b-t8",
        AttnShape(b=1, s=2048, hq=16, hkv=16, d=160, causal=True, p_drop=0.1),
        NormShape(s_local=256, b=1, h=20480, norm="layernorm", p_drop=0.1,
                  gamma="u0.9-1.1", beta="n0.02")),
    # Llama-3-70B style (h=8192, 64 q / 8 kv heads) at t=8, s=8192, GQA 8:1, no dropout
    "llama3-70b-t8": Workload(
        "llama3-70b-t8",
        AttnShape(b=1, s=8192, hq=8, hkv=1, d=128, causal=True, p_drop=0.0),
        NormShape(s_local=1024, b=1, h=8192, norm="rmsnorm", p_drop=0.0)),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 holding the bf16 value."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "fp32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(name: str, shape, seed_base: int) -> np.ndarray:
    rng = np.random.default_rng(seed_base + TENSOR_IDS[name])
    return rng.standard_normal(size=shape, dtype=np.float32)


def attn_inputs(a: AttnShape, seed_base: int = 0) -> Dict[str, np.ndarray]:
    """Q, K, V, dO for one attention-core problem (float32 arrays)."""
    out = {}
    for name, heads in (("q", a.hq), ("k", a.hkv), ("v", a.hkv), ("do", a.hq)):
        x = _normal(name, (a.b, a.s, heads, a.d), seed_base) * np.float32(a.in_scale)
        out[name] = _finish(x, a.dtype)
    return out


def norm_inputs(n: NormShape, seed_base: int = 0) -> Dict[str, np.ndarray]:
    """resid, y, du, dres ([s_local, b, h]) and gamma, beta ([h], fp32)."""
    out = {}
    for name in ("resid", "y", "du", "dres"):
        out[name] = _finish(_normal(name, (n.s_local, n.b, n.h), seed_base), n.dtype)
    if n.gamma == "ones":
        g = np.ones(n.h, np.float32)
    elif n.gamma == "u0.9-1.1":
        g = np.random.default_rng(seed_base + TENSOR_IDS["gamma"]).uniform(
            0.9, 1.1, size=n.h).astype(np.float32)
    else:
        raise ValueError(n.gamma)
    if n.beta == "zeros":
        bt = np.zeros(n.h, np.float32)
    elif n.beta == "n0.02":
        bt = _normal("beta", (n.h,), seed_base) * np.float32(0.02)
    else:
        raise ValueError(n.beta)
    out["gamma"] = g
    out["beta"] = bt
    return out
