"""Helpers for the GPU parity tests: device tensors from the seeded generator,
the error metric, and a loud failure when the GPU or the library is missing."""
import sys

import numpy as np
import pytest
import torch

from selective_recompute_attention_attn_amd import ops

# fp32 path: 1e-5; bf16 path: 2e-2 -- both as max|x - ref| / max|ref| per tensor
TOL_FP32 = 1e-5
TOL_BF16 = 2e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    ops.lib()   # raises if libsrat.so is missing
    return torch.device("cuda:0")


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), "non-finite values"
    scale = np.max(np.abs(ref))
    if scale == 0:
        return float(np.max(np.abs(x)))
    return float(np.max(np.abs(x - ref)) / scale)


def assert_close(name: str, x, ref, tol: float) -> float:
    e = rel_err(x, ref)
    assert e <= tol, f"{name}: max-norm relative error {e:.3e} > {tol:.1e}"
    return e
