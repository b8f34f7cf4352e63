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


# Rows whose largest reference value is below this fraction of the tensor's
# largest are judged against that floor instead of their own maximum (the same
# floor as the elementwise figure below): a row of near-zero values carries
# only the rounding of its larger neighbours' terms.  Rows whose reference is
# exactly zero (the first query of a causal head has one visible key, so its
# dS and dQ vanish identically, and the kernel's value there is the rounding
# of D = rowsum(dO * O) with O in bf16) have no relative error; the
# per-tensor check covers them.
ROW_FLOOR = 1e-3


def row_errs(x: np.ndarray, ref: np.ndarray, row_len: int, row_floor=None) -> np.ndarray:
    """Per-row max-norm relative error: rows are consecutive runs of row_len
    values of the C-ordered arrays (the head-dim vector of one (batch,
    position, head), or row_len = 1 for per-row scalars such as the LSE)."""
    x = np.asarray(x, np.float64).reshape(-1, row_len)
    ref = np.asarray(ref, np.float64).reshape(-1, row_len)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(x)), "non-finite values in different places"
    x = np.where(fin, x, 0.0)
    ref = np.where(fin, ref, 0.0)
    tmax = float(np.max(np.abs(ref))) if ref.size else 0.0
    if tmax == 0.0:       # an all-zero reference: absolute errors, as rel_err
        return np.max(np.abs(x), axis=1) if x.size else np.zeros(0)
    rmax = np.max(np.abs(ref), axis=1)
    den = np.maximum(rmax, ROW_FLOOR * tmax)
    if row_floor is not None:
        den = np.maximum(den, np.asarray(row_floor, np.float64).reshape(-1))
    err = np.max(np.abs(x - ref), axis=1) / den
    return np.where(rmax > 0.0, err, 0.0)


def elementwise_err(x, ref) -> float:
    """The elementwise relative figure (reported, not gated): |x - ref| over
    max(|ref|, 1e-3 max|ref|)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    x, ref = x[fin], ref[fin]
    if ref.size == 0:
        return 0.0
    den = np.maximum(np.abs(ref), ROW_FLOOR * max(float(np.max(np.abs(ref))), 1e-30))
    return float(np.max(np.abs(x - ref) / den))


def grad_term_scales(x, o_ref, lse_ref, *, causal, scale, p_drop, seed, head_offset=0, heads=None,
                     seqlens=None):
    """Per-row sizes of the terms summed into dQ and dK, from the oracle:
    ([b, s, hq] for dQ rows, [b, s, hkv] for dK rows).

    dQ_i = scale * sum_j (P_ij dP'_ij K_j - P_ij D_i K_j) and dK_j the same sum
    over queries i with Q_i (dP' = dO V^T * M / (1 - p), D_i = rowsum(dO_i *
    O_i), itself a sum of the terms dO_ie O_ie).  The size of row i is
    scale * max_d sum_j P_ij (|dP'_ij| + sum_e |dO_ie O_ie|) |K_jd|, the sum of the
    magnitudes of its terms, the bound every rounded sum is judged by.  Where the terms nearly cancel (the first queries of a causal
    head, the last keys, kept against dropped scores) a row is far smaller
    than its terms; the rounding of the bf16 operands and of the stored bf16
    O, from which any backward pass forms D, then acts at the terms' scale.
    Heads not listed stay 0; a kv-head's dK size sums over the listed
    q-heads of its group."""
    from oracle import attention as oat
    from oracle import philox as oph
    q, k, v, do = (np.asarray(x[n], np.float64) for n in ("q", "k", "v", "do"))
    o_ref = np.asarray(o_ref, np.float64)
    lse_ref = np.asarray(lse_ref, np.float64)
    b, s, hq, _ = q.shape
    hkv = k.shape[2]
    grp = hq // hkv
    lens = [s] * b if seqlens is None else [int(v) for v in seqlens]
    tq = np.zeros((b, s, hq))
    tk = np.zeros((b, s, hkv, q.shape[3]))
    for bb, hh in (heads if heads is not None else [(i, j) for i in range(b) for j in range(hq)]):
        L, g = lens[bb], hh // grp
        if L == 0:
            continue
        P = np.exp(oat.scores(q[bb, :L, hh], k[bb, :L, g], scale, causal) - lse_ref[bb, hh, :L][:, None])
        M = oph.attn_keep_mask(seed, p_drop, bb, head_offset + hh, L, L)
        dPd = (do[bb, :L, hh] @ v[bb, :L, g].T) * M / (1.0 - p_drop)
        D_abs = np.sum(np.abs(do[bb, :L, hh] * o_ref[bb, :L, hh]), axis=1)
        W = P * (np.abs(dPd) + D_abs[:, None])
        tq[bb, :L, hh] = scale * np.max(W @ np.abs(k[bb, :L, g]), axis=1)
        tk[bb, :L, g] += scale * (W.T @ np.abs(q[bb, :L, hh]))
    return tq, np.max(tk, axis=3)


def assert_close(name: str, x, ref, tol: float, row_len: int = 0, row_floor=None) -> float:
    """Per-tensor max-norm relative error within tol; with row_len > 0 also
    every row within tol (rows as in row_errs; `row_floor`, one value per row,
    raises a row's denominator to at least that value).  Returns the tensor
    figure."""
    e = rel_err(x, ref)
    assert e <= tol, f"{name}: max-norm relative error {e:.3e} > {tol:.1e}"
    if row_len:
        r = row_errs(x, ref, row_len, row_floor)
        if r.size == 0:
            return e
        worst = int(np.argmax(r))
        assert r[worst] <= tol, f"{name}: row {worst} max-norm relative error {r[worst]:.3e} > {tol:.1e}"
    return e
