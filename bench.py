#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X.

One step = attention-core forward + backward (recompute) + sequence-parallel
norm-region forward + backward, on one tensor-parallel rank's share of a
workload (default: the 22B GPT layer at t = 8), with seeded synthetic inputs
already resident in HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

ms_per_step wall clock of the K timed steps (synchronised on both sides)
value       attention-core fwd+bwd algorithmic TFLOP/s over K back-to-back
            fwd+bwd passes on the rotating buffer sets, timed by one pair of
            HIP events (timing-only, no system fence) on the launch stream;
            the norm region's GB/s likewise over K back-to-back passes each
roofline    the dominant kernel (largest share of the traced time): its
            algorithmic work per launch / its mean launch time, against
            MI355X's published peak.  Launch times come from the library's
            trace (a HIP event pair per launch, on the launch stream) in a
            second pass over the same K steps, kept out of the timed region
cpu_baseline  the float64 CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn-core fwd+bwd TFLOP/s & % bf16 MFMA peak; SP LayerNorm GB/s (1 GPU)"
PEAK_BF16_TFLOPS = 2516.6       # 256 CU x 2.4 GHz x 4096 FLOP/clk (dense)
PEAK_HBM_GBPS = 8000.0
N_SETS = 8                      # rotated input/output sets: a set's inputs have left the
                                # 256 MB last-level cache before it is used again
COPY_CALIBRATION_BYTES = 1 << 29  # 512 MiB read + 512 MiB written per calibration copy
COPY_CALIBRATION_REPS = 3


def attn_flops(a, fwd=True, bwd=True):
    """Algorithmic FLOPs: 4 (QK^T, PV) forward + 10 (QK^T recompute, dP, dV, dK, dQ)
    backward per score element and head-dim unit; causal counts half the scores."""
    units = a.b * a.hq * a.s * a.s * a.d * (0.5 if a.causal else 1.0)
    return units * ((4 if fwd else 0) + (10 if bwd else 0))


def norm_bytes(n, fwd=True):
    """Algorithmic HBM bytes: fwd reads resid, y and writes h, u; bwd reads du, dres, h
    and writes dh, dy (dy is dh when p = 0); plus per-row statistics and [h] vectors."""
    e = 2 if n.dtype == "bf16" else 4
    elems = n.rows * n.h
    stats = n.rows * (8 if n.norm == "layernorm" else 4)
    vecs = n.h * 4 * (2 if n.norm == "layernorm" else 1)
    if fwd:
        return elems * 4 * e + stats + vecs
    tensors = 5 if n.p_drop > 0 else 4
    return elems * tensors * e + stats + 2 * vecs


# Algorithmic FLOPs per score element and head-dim unit of each attention
# kernel: forward QK^T + PV = 4; backward 10 = QK^T recompute, dP, dV, dK (the
# dK/dV kernel, 8) + dQ (the dQ kernel, 2; the QK^T and dO V^T it re-does to
# avoid atomics are not algorithmic work).
KERNEL_FLOP_UNITS = {"attn_fwd_bf16": 4, "attn_bwd_dkdv": 8, "attn_bwd_dq": 2}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since it was taken."""
    from selective_recompute_attention_attn_amd import profiling
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path) or kernel not in profiling.KERNEL_SOURCES:
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != profiling.src_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, seconds_budget=15.0):
    """Time the float64 oracle on a bounded sample: (batch, head) pairs of the
    attention core (fwd + recompute bwd) until about `seconds_budget` seconds of
    CPU work have been spent, and some rows of the norm region."""
    import numpy as np
    from oracle import attention as oat
    from oracle import norm as onm
    from selective_recompute_attention_attn_amd import gen
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        blas_threads = None
    a, n = w.attn, w.norm
    x = gen.attn_inputs(a)
    kw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed)
    heads, t_attn = [], 0.0
    for bb in range(a.b):
        for hh in range(a.hq):
            t0 = time.perf_counter()
            o, lse = oat.attn_fwd(x["q"], x["k"], x["v"], heads=[(bb, hh)], **kw)
            oat.attn_bwd(x["q"], x["k"], x["v"], lse, x["do"], heads=[(bb, hh)], **kw)
            t_attn += time.perf_counter() - t0
            heads.append((bb, hh))
            if t_attn > seconds_budget * 0.8:
                break
        if t_attn > seconds_budget * 0.8:
            break
    per_head = attn_flops(a) / (a.b * a.hq)
    tflops = per_head * len(heads) / t_attn / 1e12
    y = gen.norm_inputs(n)
    rows = max(1, min(n.s_local, 64))
    nkw = dict(norm=n.norm, p_drop=n.p_drop, seed=n.seed, site=n.site)
    t0 = time.perf_counter()
    h, u, mu, rs = onm.sp_norm_fwd(y["resid"][:rows], y["y"][:rows], y["gamma"], y["beta"], eps=n.eps, **nkw)
    onm.sp_norm_bwd(y["du"][:rows], y["dres"][:rows], h, y["gamma"], mu, rs, **nkw)
    t_norm = time.perf_counter() - t0
    sub = n.with_(s_local=rows)
    gbps = (norm_bytes(sub, True) + norm_bytes(sub, False)) / t_norm / 1e9
    return {"value": tflops, "unit": "TFLOP/s", "cores": blas_threads or len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{len(heads)} of {a.b * a.hq} (batch, q-head) pairs: attention fwd + recompute bwd in "
                      f"float64 numpy with the full {a.s}x{a.s} score matrix ({t_attn:.1f} s; BLAS threads "
                      f"{blas_threads}, elementwise single-threaded); norm region {rows * n.b} of {n.rows} rows "
                      f"fwd+bwd at {gbps:.3f} GB/s",
            "norm_gbps": gbps, "host_cores": len(os.sched_getaffinity(0))}


class TimingEvent:
    """HIP event used for timing only, created with hipEventDisableSystemFence:
    recording it adds no system-scope cache writeback / invalidation between
    the kernels it brackets (torch's events do)."""
    _hip = None

    def __init__(self, stream: int):
        if TimingEvent._hip is None:
            h = ctypes.CDLL("libamdhip64.so.7")   # the HIP runtime torch has loaded
            vp = ctypes.c_void_p
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            h.hipEventDestroy.argtypes = [vp]
            TimingEvent._hip = h
        self.ev = ctypes.c_void_p()
        self.stream = ctypes.c_void_p(stream)
        if TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), 0x20000000) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self) -> None:
        if TimingEvent._hip.hipEventRecord(self.ev, self.stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end: "TimingEvent") -> float:
        ms = ctypes.c_float(0.0)
        if TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and self.ev:
            TimingEvent._hip.hipEventDestroy(self.ev)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt22b-t8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true", help="skip the traced pass (per-kernel durations)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="before warmup, run COPY_CALIBRATION_REPS plain device copies of "
                         "COPY_CALIBRATION_BYTES (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_recompute_attention_attn_amd import gen, ops

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    ops.lib()
    dev = torch.device("cuda:0")
    w = gen.WORKLOADS[args.workload]
    a, n = w.attn, w.norm
    tdt = torch.bfloat16 if a.dtype == "bf16" else torch.float32
    ndt = torch.bfloat16 if n.dtype == "bf16" else torch.float32

    def t(x, dt):
        return torch.from_numpy(x).to(dt).to(dev)

    xa = gen.attn_inputs(a)
    xn = gen.norm_inputs(n)
    sets = []
    for _ in range(N_SETS):
        s = {k: t(xa[k], tdt) for k in ("q", "k", "v", "do")}
        s["o"] = torch.empty_like(s["q"])
        s["lse"] = torch.empty((a.b, a.hq, a.s), dtype=torch.float32, device=dev)
        s["grads"] = (torch.empty_like(s["q"]), torch.empty_like(s["k"]), torch.empty_like(s["v"]))
        for k in ("resid", "y", "du", "dres"):
            s[k] = t(xn[k], ndt)
        s["gamma"] = torch.tensor(xn["gamma"], device=dev)
        s["beta"] = torch.tensor(xn["beta"], device=dev)
        ln = n.norm == "layernorm"
        s["nf"] = (torch.empty_like(s["resid"]), torch.empty_like(s["resid"]),
                   torch.empty(n.rows, dtype=torch.float32, device=dev) if ln else None,
                   torch.empty(n.rows, dtype=torch.float32, device=dev))
        dh = torch.empty_like(s["resid"])
        s["nb"] = (dh, dh if n.p_drop == 0 else torch.empty_like(s["resid"]),
                   torch.empty(n.h, dtype=torch.float32, device=dev),
                   torch.empty(n.h, dtype=torch.float32, device=dev) if ln else None)
        sets.append(s)
    desc = ops.attn_desc(sets[0]["q"], sets[0]["k"], sets[0]["v"], sets[0]["o"], causal=a.causal,
                         scale=a.scale, p_drop=a.p_drop, seed=a.seed, head_offset=0)
    ws_attn = torch.empty(ops.attn_bwd_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    need_f = ops.attn_fwd_workspace_bytes(desc)
    ws_fwd = torch.empty(need_f, dtype=torch.uint8, device=dev) if need_f else None
    ndesc = ops.norm_desc(sets[0]["resid"], norm=n.norm, eps=n.eps, p_drop=n.p_drop, seed=n.seed, site=n.site,
                          seq_offset=0)
    need = ops.sp_norm_bwd_workspace_bytes(ndesc)
    ws_norm = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    akw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed)
    nkw = dict(norm=n.norm, p_drop=n.p_drop, seed=n.seed, site=n.site)

    # every call marshalled once per buffer set: the timed loop issues one foreign
    # call per library entry point, so the host stays ahead of the GPU
    calls = []
    for s in sets:
        h, u, mu, rs = s["nf"]
        calls.append((
            ops.prepare_attn_fwd(s["q"], s["k"], s["v"], s["o"], s["lse"], workspace=ws_fwd, **akw),
            ops.prepare_attn_bwd(s["q"], s["k"], s["v"], s["o"], s["lse"], s["do"], *s["grads"], ws_attn,
                                 **akw),
            ops.prepare_sp_norm_fwd(s["resid"], s["y"], s["gamma"], s["beta"], h, u, mu, rs, eps=n.eps, **nkw),
            ops.prepare_sp_norm_bwd(s["du"], s["dres"], h, s["gamma"], mu, rs, *s["nb"], ws_norm, **nkw)))

    def step(i):
        fwd, bwd, nfwd, nbwd = calls[i % N_SETS]
        fwd()
        bwd()
        nfwd()
        nbwd()

    def attn_pass(i):
        fwd, bwd, _, _ = calls[i % N_SETS]
        fwd()
        bwd()

    def norm_fwd_pass(i):
        calls[i % N_SETS][2]()

    def norm_bwd_pass(i):
        calls[i % N_SETS][3]()

    def region_ms(fn, k):
        """Mean time of one of k back-to-back calls of fn, from one event pair
        on the launch stream: a timing event recorded between kernels leaves
        the GPU idle for a few microseconds, so none sits inside the region."""
        ev0, ev1 = TimingEvent(stream), TimingEvent(stream)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(k):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / k

    if args.calibrate_copy:
        src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(COPY_CALIBRATION_REPS):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev).cuda_stream
    # the K timed steps (wall clock, synchronised on both sides)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the attention core and the norm region, each as K back-to-back passes
    # over the same rotating buffer sets
    attn_ms = region_ms(attn_pass, args.steps)
    nf_ms = region_ms(norm_fwd_pass, args.steps)
    nb_ms = region_ms(norm_bwd_pass, args.steps)
    # per-kernel durations come from a second pass over the same K steps with
    # the library's launch trace on: its two events per launch add a few
    # microseconds between kernels, so they stay out of the timed region above
    trace = {}
    if not args.no_trace:
        ops.trace_enable(True)
        ops.trace_read(reset=True)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        trace = ops.trace_read(reset=True)
        ops.trace_enable(False)
    ms_step = (t1 - t0) * 1e3 / args.steps
    flops = attn_flops(a)
    value = flops / (attn_ms * 1e-3) / 1e12

    kernels = {k: {"launches": v[0], "mean_us": 1e3 * v[1] / max(v[0], 1)} for k, v in trace.items()}
    roofline = None
    if kernels:
        dom = max(trace, key=lambda k: trace[k][1])
        mean_s = trace[dom][1] / trace[dom][0] * 1e-3
        units = a.b * a.hq * a.s * a.s * a.d * (0.5 if a.causal else 1.0)
        work = {k: ("mfma", units * u) for k, u in KERNEL_FLOP_UNITS.items()}
        work.update({"sp_norm_fwd": ("hbm", norm_bytes(n, True)),
                     "sp_norm_bwd": ("hbm", norm_bytes(n, False))})
        if dom in work:
            bound, amount = work[dom]
            if bound == "mfma":
                achieved, peak, unit = amount / mean_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
            else:
                achieved, peak, unit = amount / mean_s / 1e9, PEAK_HBM_GBPS, "GB/s"
            roofline = {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                        "frac": achieved / peak, "traffic": measured_traffic(dom, w.name),
                        "mean_launch_us": mean_s * 1e6}

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": a.dtype, "data": "synthetic",
        "config": {"workload": w.name, "b": a.b, "s": a.s, "hq": a.hq, "hkv": a.hkv, "d": a.d,
                   "causal": a.causal, "p_attn": a.p_drop, "norm": n.norm, "norm_rows": n.rows, "h": n.h,
                   "p_hidden": n.p_drop, "parallelism": "one tensor-parallel rank (t=8) on 1 GPU"},
        "attn_frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
        "attn_ms": attn_ms,
        "attn_fwd_tflops": (attn_flops(a, True, False) / (kernels["attn_fwd_bf16"]["mean_us"] * 1e-6) / 1e12
                            if "attn_fwd_bf16" in kernels else None),
        "attn_bwd_tflops": (attn_flops(a, False, True)
                            / (sum(v["mean_us"] for k, v in kernels.items() if k.startswith("attn_bwd")) * 1e-6)
                            / 1e12 if "attn_bwd_dkdv" in kernels else None),
        "sp_fwd_gbps": norm_bytes(n, True) / (nf_ms * 1e-3) / 1e9,
        "sp_bwd_gbps": norm_bytes(n, False) / (nb_ms * 1e-3) / 1e9,
        "sp_fwd_frac_of_hbm": norm_bytes(n, True) / (nf_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "sp_bwd_frac_of_hbm": norm_bytes(n, False) / (nb_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
