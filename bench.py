#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X.

One step = attention-core forward + backward (recompute) + sequence-parallel
norm-region forward + backward, on one tensor-parallel rank's share of a
workload, with seeded synthetic inputs already resident in HBM.  The headline
workload is the largest single-GPU one, the Llama-3-70B-style rank
(llama3-70b-t8: s 8192, 8 q-heads on 1 kv-head of 128, causal, RMSNorm region
of 1024 x 8192); the three GPT-style ranks are measured in the same run as
sub-results.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--sub NAME,NAME | --sub none] [--no-cpu-baseline]

ms_per_step   wall clock of the K timed steps of the headline workload
              (synchronised on both sides); before the W warm-up steps each
              workload runs its own steps untimed for 0.25 s, so that the
              GPU clocks have settled
value         attention-core fwd+bwd algorithmic TFLOP/s of the headline
              workload over K back-to-back fwd+bwd passes on rotating buffer
              sets, timed by one pair of HIP events (timing-only, no system
              fence) on the launch stream
timing        median / p10 / p90 over K passes, each bracketed by its own
              event pair (fwd, bwd and fwd+bwd; each pass carries one event
              gap of a few microseconds, so these sit slightly above `value`'s)
roofline      the dominant kernel (largest share of the traced time): its
              algorithmic work per launch / its mean launch time (a HIP event
              pair per launch on the launch stream, in a separate traced pass)
cpu_baseline  the float64 CPU oracle on a bounded sample of the headline
              workload: forward and backward seconds, GFLOP/s at the oracle's
              dense work and at the algorithmic work, and the parity errors
              of the GPU outputs on the sampled heads
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
SETTLE_S = 0.25                 # seconds of untimed steps before each workload's warm-up steps
HEADLINE = "llama3-70b-t8"
SUBS = ("gpt22b-t8", "gpt175b-t8", "gpt530b-t8")
LARGEST_LAYERNORM = "gpt22b-t8"  # 1024 x 6144 rows: the largest LayerNorm region of the workloads


def attn_units(a):
    return a.b * a.hq * a.s * a.s * a.d * (0.5 if a.causal else 1.0)


def attn_flops(a, fwd=True, bwd=True):
    """Algorithmic FLOPs: 4 (QK^T, PV) forward + 10 (QK^T recompute, dP, dV, dK, dQ)
    backward per score element and head-dim unit; causal counts half the scores."""
    return attn_units(a) * ((4 if fwd else 0) + (10 if bwd else 0))


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


def _pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    k = (len(xs) - 1) * q
    lo = int(k)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def _dist(xs):
    return {"median_ms": _pct(xs, 0.5), "p10_ms": _pct(xs, 0.1), "p90_ms": _pct(xs, 0.9), "reps": len(xs)}


def cpu_baseline(w, got, seconds_budget=15.0):
    """Time the float64 oracle on a bounded sample of (batch, q-head) pairs of the
    attention core -- forward and recompute backward timed separately -- until
    about `seconds_budget` seconds of CPU work are spent, plus some rows of the
    norm region; compare the GPU outputs `got` (set 0) on the sampled heads."""
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
    heads, t_fwd, t_bwd = [], 0.0, 0.0
    ref, kv_ref = {}, {}
    order = [(bb, hh) for bb in range(a.b) for hh in range(a.hq)]
    # spread the sample over batch elements and heads
    order = order[::max(1, len(order) // 8)] + [p for p in order if p not in order[::max(1, len(order) // 8)]]
    for bb, hh in order:
        t0 = time.perf_counter()
        o, lse = oat.attn_fwd(x["q"], x["k"], x["v"], heads=[(bb, hh)], **kw)
        t1 = time.perf_counter()
        dq, dk, dv = oat.attn_bwd(x["q"], x["k"], x["v"], lse, x["do"], heads=[(bb, hh)], **kw)
        t2 = time.perf_counter()
        t_fwd += t1 - t0
        t_bwd += t2 - t1
        heads.append((bb, hh))
        g = hh // (a.hq // a.hkv)
        ref[(bb, hh)] = (o[bb, :, hh], lse[bb, hh], dq[bb, :, hh])
        # a kv-head's dK / dV sum the contributions of its q-heads
        kv_ref[(bb, g)] = kv_ref.get((bb, g), 0) + np.stack([dk[bb, :, g], dv[bb, :, g]])
        if t_fwd + t_bwd > seconds_budget:
            break
    per_head = attn_units(a) / (a.b * a.hq)
    dense_per_head = a.s * a.s * a.d          # the oracle materialises every score, causal or not
    t_all = t_fwd + t_bwd
    nh = len(heads)

    # parity of the GPU outputs on the sampled heads (max-norm relative per
    # tensor); dK / dV of a kv-head sum over every q-head of its group, so
    # they are compared on the kv-heads whose whole group was sampled
    def rel(g, r):
        g = np.asarray(g, np.float64)
        r = np.asarray(r, np.float64)
        return float(np.max(np.abs(g - r)) / max(float(np.max(np.abs(r))), 1e-30))
    parity = {}
    if got is not None:
        grp = a.hq // a.hkv
        for i, name in enumerate(("o", "lse", "dq")):
            gs = [got[name][bb, hh] if name == "lse" else got[name][bb, :, hh] for bb, hh in heads]
            parity[name] = rel(np.stack(gs), np.stack([ref[p][i] for p in heads]))
        whole = [(bb, g) for (bb, g) in kv_ref
                 if all((bb, g * grp + j) in ref for j in range(grp))]
        for i, name in enumerate(("dk", "dv")):
            parity[name] = (rel(np.stack([got[name][bb, :, g] for bb, g in whole]),
                                np.stack([kv_ref[p][i] for p in whole])) if whole else None)
        parity["kv_heads_compared"] = len(whole)
    y = gen.norm_inputs(n)
    rows = max(1, min(n.s_local, 64))
    nkw = dict(norm=n.norm, p_drop=n.p_drop, seed=n.seed, site=n.site)
    t0 = time.perf_counter()
    h, u, mu, rs_ = onm.sp_norm_fwd(y["resid"][:rows], y["y"][:rows], y["gamma"], y["beta"], eps=n.eps, **nkw)
    onm.sp_norm_bwd(y["du"][:rows], y["dres"][:rows], h, y["gamma"], mu, rs_, **nkw)
    t_norm = time.perf_counter() - t0
    sub = n.with_(s_local=rows)
    gbps = (norm_bytes(sub, True) + norm_bytes(sub, False)) / t_norm / 1e9
    return {"value": attn_flops(a) / (a.b * a.hq) * nh / t_all / 1e12, "unit": "TFLOP/s",
            "cores": blas_threads or len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{nh} of {a.b * a.hq} (batch, q-head) pairs of {w.name}: attention fwd + recompute bwd in "
                      f"float64 numpy with the full {a.s}x{a.s} score matrix ({t_all:.1f} s; BLAS threads "
                      f"{blas_threads}, elementwise single-threaded); norm region {rows * n.b} of {n.rows} rows "
                      f"fwd+bwd",
            "fwd_s": t_fwd, "bwd_s": t_bwd, "pairs": nh,
            "fwd_gflops_algorithmic": 4 * per_head * nh / t_fwd / 1e9,
            "bwd_gflops_algorithmic": 10 * per_head * nh / t_bwd / 1e9,
            "fwd_gflops_dense": 4 * dense_per_head * nh / t_fwd / 1e9,
            "bwd_gflops_dense": 10 * dense_per_head * nh / t_bwd / 1e9,
            "parity_max_rel": parity,
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


class Bench:
    """Rotating buffer sets of one workload with every library call marshalled
    once per set (ops.prepare_*): the timed loops issue one foreign call per
    entry point, so the host stays ahead of the GPU."""

    def __init__(self, w, dev):
        import torch
        from selective_recompute_attention_attn_amd import gen, ops
        self.torch, self.ops, self.w, self.dev = torch, ops, w, dev
        a, n = w.attn, w.norm
        tdt = torch.bfloat16 if a.dtype == "bf16" else torch.float32
        ndt = torch.bfloat16 if n.dtype == "bf16" else torch.float32

        def t(x, dt):
            return torch.from_numpy(x).to(dt).to(dev)

        xa = gen.attn_inputs(a)
        xn = gen.norm_inputs(n)
        self.sets = []
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
            self.sets.append(s)
        s0 = self.sets[0]
        desc = ops.attn_desc(s0["q"], s0["k"], s0["v"], s0["o"], causal=a.causal, scale=a.scale,
                             p_drop=a.p_drop, seed=a.seed, head_offset=0)
        self.ws_attn = torch.empty(ops.attn_bwd_workspace_bytes(desc), dtype=torch.uint8, device=dev)
        need_f = ops.attn_fwd_workspace_bytes(desc)
        self.ws_fwd = torch.empty(need_f, dtype=torch.uint8, device=dev) if need_f else None
        ndesc = ops.norm_desc(s0["resid"], norm=n.norm, eps=n.eps, p_drop=n.p_drop, seed=n.seed, site=n.site,
                              seq_offset=0)
        need = ops.sp_norm_bwd_workspace_bytes(ndesc)
        self.ws_norm = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        akw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed)
        nkw = dict(norm=n.norm, p_drop=n.p_drop, seed=n.seed, site=n.site)
        self.calls = []
        for s in self.sets:
            h, u, mu, rs = s["nf"]
            self.calls.append((
                ops.prepare_attn_fwd(s["q"], s["k"], s["v"], s["o"], s["lse"], workspace=self.ws_fwd, **akw),
                ops.prepare_attn_bwd(s["q"], s["k"], s["v"], s["o"], s["lse"], s["do"], *s["grads"],
                                     self.ws_attn, **akw),
                ops.prepare_sp_norm_fwd(s["resid"], s["y"], s["gamma"], s["beta"], h, u, mu, rs, eps=n.eps,
                                        **nkw),
                ops.prepare_sp_norm_bwd(s["du"], s["dres"], h, s["gamma"], mu, rs, *s["nb"], self.ws_norm,
                                        **nkw)))
        self.stream = torch.cuda.current_stream(dev).cuda_stream

    def step(self, i):
        for c in self.calls[i % N_SETS]:
            c()

    def region_ms(self, which, k):
        """Mean time of one of k back-to-back calls (entry points `which`), from
        one event pair on the launch stream: a timing event recorded between
        kernels leaves the GPU idle for a few microseconds, so none sits
        inside the region."""
        ev0, ev1 = TimingEvent(self.stream), TimingEvent(self.stream)
        self.torch.cuda.synchronize()
        ev0.record()
        for i in range(k):
            for j in which:
                self.calls[i % N_SETS][j]()
        ev1.record()
        self.torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / k

    def per_pass(self, k):
        """k attention passes, each bracketed by events: fwd, bwd, fwd+bwd times (ms)."""
        evs = [[TimingEvent(self.stream) for _ in range(3)] for _ in range(k)]
        self.torch.cuda.synchronize()
        for i in range(k):
            fwd, bwd = self.calls[i % N_SETS][:2]
            evs[i][0].record()
            fwd()
            evs[i][1].record()
            bwd()
            evs[i][2].record()
        self.torch.cuda.synchronize()
        f = [e[0].elapsed_time(e[1]) for e in evs]
        b = [e[1].elapsed_time(e[2]) for e in evs]
        return f, b, [x + y for x, y in zip(f, b)]

    def traced(self, k):
        ops = self.ops
        ops.trace_enable(True)
        ops.trace_read(reset=True)
        for i in range(k):
            self.step(i)
        self.torch.cuda.synchronize()
        trace = ops.trace_read(reset=True)
        ops.trace_enable(False)
        return trace

    def settle(self, seconds=SETTLE_S):
        """Runs the workload's own steps, untimed, for a fraction of a second
        before the warm-up steps.  The GPU's clocks take some 30-40 ms of
        this work to reach their steady level (launches before that run up
        to 25 % slower, also right after other heavy work), so the timed
        steps, and a profiler's per-kernel mean over the whole run, see the
        steady clocks."""
        t0, i = time.perf_counter(), 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(N_SETS):
                self.step(i)
                i += 1
            self.torch.cuda.synchronize()
        return i

    def measure(self, steps, warmup, trace=True):
        a, n = self.w.attn, self.w.norm
        self.settle()
        for i in range(warmup):
            self.step(i)
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        self.torch.cuda.synchronize()
        t1 = time.perf_counter()
        attn_ms = self.region_ms((0, 1), steps)
        fwd_ms = self.region_ms((0,), steps)
        bwd_ms = self.region_ms((1,), steps)
        nf_ms = self.region_ms((2,), steps)
        nb_ms = self.region_ms((3,), steps)
        pf, pb, pfb = self.per_pass(steps)
        tr = self.traced(steps) if trace else {}
        kernels = {k: {"launches": v[0], "mean_us": 1e3 * v[1] / max(v[0], 1)} for k, v in tr.items()}
        value = attn_flops(a) / (attn_ms * 1e-3) / 1e12
        r = {
            "workload": self.w.name, "value": value, "frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
            "ms_per_step": (t1 - t0) * 1e3 / steps, "attn_ms": attn_ms,
            "attn_fwd_ms": fwd_ms, "attn_bwd_ms": bwd_ms,
            "attn_fwd_tflops": attn_flops(a, True, False) / (fwd_ms * 1e-3) / 1e12,
            "attn_bwd_tflops": attn_flops(a, False, True) / (bwd_ms * 1e-3) / 1e12,
            "timing": {"fwd": _dist(pf), "bwd": _dist(pb), "fwd_bwd": _dist(pfb)},
            "norm": n.norm, "sp_fwd_gbps": norm_bytes(n, True) / (nf_ms * 1e-3) / 1e9,
            "sp_bwd_gbps": norm_bytes(n, False) / (nb_ms * 1e-3) / 1e9,
            "kernels": kernels,
        }
        r["sp_fwd_frac_of_hbm"] = r["sp_fwd_gbps"] / PEAK_HBM_GBPS
        r["sp_bwd_frac_of_hbm"] = r["sp_bwd_gbps"] / PEAK_HBM_GBPS
        r["roofline"] = self.roofline(tr)
        return r

    def roofline(self, tr):
        if not tr:
            return None
        a, n = self.w.attn, self.w.norm
        dom = max(tr, key=lambda k: tr[k][1])
        mean_s = tr[dom][1] / tr[dom][0] * 1e-3
        work = {k: ("mfma", attn_units(a) * u) for k, u in KERNEL_FLOP_UNITS.items()}
        work.update({"sp_norm_fwd": ("hbm", norm_bytes(n, True)), "sp_norm_bwd": ("hbm", norm_bytes(n, False))})
        if dom not in work:
            return None
        bound, amount = work[dom]
        if bound == "mfma":
            achieved, peak, unit = amount / mean_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        else:
            achieved, peak, unit = amount / mean_s / 1e9, PEAK_HBM_GBPS, "GB/s"
        return {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": measured_traffic(dom, self.w.name),
                "mean_launch_us": mean_s * 1e6, "work_per_launch": amount}

    def outputs_set0(self):
        """Host copies of set 0's forward and backward outputs (after the runs above)."""
        s = self.sets[0]
        self.calls[0][0]()
        self.calls[0][1]()
        self.torch.cuda.synchronize()
        f = lambda t: t.detach().float().cpu().numpy()
        return {"o": f(s["o"]), "lse": f(s["lse"]), "dq": f(s["grads"][0]), "dk": f(s["grads"][1]),
                "dv": f(s["grads"][2])}


def no_s2_alloc(w, dev):
    """Peak device-memory growth of one fwd+bwd call through the binding, less
    the call's own outputs (O, LSE, dQ, dK, dV), against the size of one bf16
    s x s score matrix per (batch, q-head): what the path needs beyond its
    outputs (its workspaces) stays below one score matrix."""
    import torch
    from selective_recompute_attention_attn_amd import ops
    a = w.attn
    g = torch.Generator(device="cpu").manual_seed(0)
    q = (torch.randn(a.b, a.s, a.hq, a.d, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    kv = (torch.randn(a.b, a.s, a.hkv, a.d, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    kw = dict(causal=a.causal, scale=a.scale, p_drop=a.p_drop, seed=a.seed)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    o, lse = ops.attn_core_fwd(q, kv, kv, **kw)
    grads = ops.attn_core_bwd(q, kv, kv, o, lse, q, **kw)
    torch.cuda.synchronize()
    growth = torch.cuda.max_memory_allocated(dev) - base
    outs = sum(t.numel() * t.element_size() for t in (o, lse, *grads))
    s2 = a.b * a.hq * a.s * a.s * 2
    del o, lse, grads
    return {"peak_growth_bytes": int(growth), "output_bytes": int(outs), "bf16_s2_bytes": int(s2),
            "ok": bool(growth - outs < s2)}


def mask_bitexact(dev, name="gpt22b-t8"):
    """The library's attention keep mask (the device function the kernels
    use) against the oracle's, for every batch element of two heads of a
    dropout workload."""
    import numpy as np
    from oracle import philox as oph
    from selective_recompute_attention_attn_amd import gen, ops
    a = gen.WORKLOADS[name].attn
    ok = True
    for hh in (0, a.hq - 1):
        m = ops.attn_dropout_mask(a.b, a.s, 1, p_drop=a.p_drop, seed=a.seed, head_offset=a.head_offset + hh,
                                  device=dev).cpu().numpy()
        for bb in range(a.b):
            ref = oph.attn_keep_mask(a.seed, a.p_drop, bb, a.head_offset + hh, a.s, a.s)
            ok = ok and bool(np.array_equal(m[bb, 0].astype(bool), ref))
    return {"workload": name, "heads": [0, a.hq - 1], "batch_elements": a.b, "ok": ok}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--sub", default=",".join(SUBS),
                    help="comma-separated workloads measured as sub-results, or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-checks", action="store_true", help="skip the mask and allocation checks")
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

    if args.calibrate_copy:
        src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(COPY_CALIBRATION_REPS):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    bench = Bench(w, dev)
    head = bench.measure(args.steps, args.warmup, trace=not args.no_trace)
    got = bench.outputs_set0() if not args.no_cpu_baseline else None
    del bench
    torch.cuda.empty_cache()

    subs = {}
    names = [] if args.sub in ("", "none") else [s for s in args.sub.split(",") if s != w.name]
    for name in names:
        b = Bench(gen.WORKLOADS[name], dev)
        r = b.measure(args.steps, args.warmup, trace=not args.no_trace)
        del b
        torch.cuda.empty_cache()
        subs[name] = r

    ln = head if n.norm == "layernorm" else subs.get(LARGEST_LAYERNORM)
    out = {
        "metric": METRIC, "value": head["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": a.dtype, "data": "synthetic",
        "config": {"workload": w.name, "b": a.b, "s": a.s, "hq": a.hq, "hkv": a.hkv, "d": a.d,
                   "causal": a.causal, "p_attn": a.p_drop, "norm": n.norm, "norm_rows": n.rows, "h": n.h,
                   "p_hidden": n.p_drop, "parallelism": "one tensor-parallel rank (t=8) on 1 GPU"},
        "attn_frac_of_bf16_peak": head["frac_of_bf16_peak"],
        "attn_ms": head["attn_ms"],
        "attn_fwd_tflops": head["attn_fwd_tflops"],
        "attn_bwd_tflops": head["attn_bwd_tflops"],
        "timing": head["timing"],
        "sp_layernorm_gbps": None if ln is None else {
            "workload": ln["workload"], "fwd": ln["sp_fwd_gbps"], "bwd": ln["sp_bwd_gbps"],
            "fwd_frac_of_hbm": ln["sp_fwd_frac_of_hbm"], "bwd_frac_of_hbm": ln["sp_bwd_frac_of_hbm"]},
        "sp_norm_gbps": {"workload": w.name, "norm": n.norm, "fwd": head["sp_fwd_gbps"],
                         "bwd": head["sp_bwd_gbps"], "fwd_frac_of_hbm": head["sp_fwd_frac_of_hbm"],
                         "bwd_frac_of_hbm": head["sp_bwd_frac_of_hbm"]},
        "kernels": head["kernels"],
        "roofline": head["roofline"],
        "sub_results": subs,
        "mask_bitexact": None,
        "no_s2_alloc": None,
        "cpu_baseline": None,
    }
    if not args.no_checks:
        out["mask_bitexact"] = mask_bitexact(dev)
        out["no_s2_alloc"] = no_s2_alloc(w, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, got)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
