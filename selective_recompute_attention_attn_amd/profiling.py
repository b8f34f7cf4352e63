"""Summaries of rocprofv3 output for the library's kernels.

Three summaries, written as short text files:

* ``stats``   -- a ``--kernel-trace --stats`` run: per-kernel call count and
  mean / min / max duration, as a markdown table.
* ``traffic`` -- two ``--pmc`` runs of the same command, one collecting
  ``FETCH_SIZE`` and one ``WRITE_SIZE`` (KiB per dispatch).  Each counter is
  scaled by the factor that makes it read the known size of a plain device
  copy launched in the same run (bench.py ``--calibrate-copy``), and the
  per-launch HBM bytes of every library kernel are written as JSON together
  with a hash of the kernel's sources, so that a later change of the kernel
  invalidates the figure.
* ``counters`` -- several ``--pmc`` passes of SQ/GRBM counters: per-kernel
  instruction counts and unit busy / wave wait shares, as a markdown table.

    python -m selective_recompute_attention_attn_amd.profiling stats \\
        --csv <dir>/run_kernel_stats.csv --workload gpt22b-t8 --command "..."
    python -m selective_recompute_attention_attn_amd.profiling traffic \\
        --fetch <dir>/f_counter_collection.csv --write <dir>/w_counter_collection.csv \\
        --workload gpt22b-t8 --command-fetch "..." --command-write "..."
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = "selective_recompute_attention_attn_amd/csrc/"
_COMMON = [CSRC + "philox.hpp", CSRC + "common.hpp", CSRC + "kernels.hpp"]
_BWD = [CSRC + "attn_bwd.hip"] + _COMMON
_NORM = [CSRC + "sp_norm.hip"] + _COMMON

# library trace name (kernel name without "_kernel") -> the sources it is built from
KERNEL_SOURCES = {
    "attn_fwd_bf16": [CSRC + "attn_fwd.hip"] + _COMMON,
    "attn_bwd_dkdv": _BWD,
    "attn_bwd_dq": _BWD,
    "attn_bwd_sums": _BWD,
    "attn_fwd_merge": [CSRC + "attn_fwd.hip"] + _COMMON,
    "sp_norm_fwd": _NORM,
    "sp_norm_bwd": _NORM,
}

# bench.py --calibrate-copy: each copy reads and writes this many bytes
COPY_BYTES = 1 << 29
COPY_PATTERN = re.compile(r"copy", re.I)


def src_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _mangled(full: str):
    """(kernel name, template arguments) of an Itanium-mangled name in namespace
    srat's anonymous namespace (left mangled when the tool cannot demangle
    __bf16 template arguments), else None."""
    m = re.match(r"_ZN4srat12_GLOBAL__N_1(\d+)", full)
    if not m:
        return None
    n = int(m.group(1))
    name = full[m.end():m.end() + n]
    rest = full[m.end() + n:]
    args = []
    if rest.startswith("I"):
        for tok in re.finditer(r"DF16b|Li(\d+)E|Lb([01])E|[A-Za-z]", rest[1:]):
            if tok.group(0) == "DF16b":
                args.append("bf16")
            elif tok.group(1) is not None:
                args.append(tok.group(1))
            elif tok.group(2) is not None:
                args.append("true" if tok.group(2) == "1" else "false")
            elif tok.group(0) == "f":
                args.append("float")
            elif tok.group(0) == "E":
                break
    return name, args


# kernels that the library's trace reports under another entry's name: the
# two-group forward and dQ kernels and the producer/consumer dK/dV kernel
# (d = 128, 160) stand in for the one-group kernels there
TRACE_ALIASES = {"attn_fwd_pp": "attn_fwd_bf16", "attn_bwd_dq_pp": "attn_bwd_dq", "attn_bwd_dkdv_pc": "attn_bwd_dkdv"}


def short_name(full: str) -> str:
    """'void srat::(anonymous namespace)::attn_bwd_dq_kernel<96, true>(srat::AttnParams)'
    (or its mangled form) -> 'attn_bwd_dq', the name the library's own trace
    uses; names of other kernels are returned unchanged."""
    mg = _mangled(full)
    if mg and mg[0].endswith("_kernel"):
        k = mg[0][:-len("_kernel")]
        return TRACE_ALIASES.get(k, k)
    m = (re.search(r"srat::(?:\(anonymous namespace\)::)?([A-Za-z0-9_]+?)_kernel\b", full)
         or re.match(r"([A-Za-z0-9_]+?)_kernel\(", full))
    return TRACE_ALIASES.get(m.group(1), m.group(1)) if m else full


def pretty_name(full: str) -> str:
    mg = _mangled(full)
    if mg:
        return f"{mg[0]}<{', '.join(mg[1])}>" if mg[1] else mg[0]
    nm = re.sub(r"^void ", "", full).replace("srat::(anonymous namespace)::", "")
    nm = re.sub(r"\(srat::[A-Za-z]+\)$", "", nm)
    return re.sub(r"_kernel\(.*\)$", "_kernel", nm)


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(names)


def stats_table(path: str):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = _col(r, "Name", "KernelName", "Kernel_Name")
            calls = int(_col(r, "Calls"))
            ns_avg = float(_col(r, "AverageNs", "Average_Ns"))
            ns_min = float(_col(r, "MinNs", "Min_Ns"))
            ns_max = float(_col(r, "MaxNs", "Max_Ns"))
            pct = float(_col(r, "Percentage"))
            rows.append((name, calls, ns_avg / 1e3, ns_min / 1e3, ns_max / 1e3, pct))
    return rows


def counter_per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} (rows of one dispatch are summed)."""
    per = collections.defaultdict(float)
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if _col(r, "Counter_Name", "Counter-Name") != counter:
                continue
            d = _col(r, "Dispatch_Id", "Dispatch-Id")
            per[d] += float(_col(r, "Counter_Value", "Counter-Value"))
            names[d] = _col(r, "Kernel_Name", "Kernel-Name")
    out = collections.defaultdict(list)
    for d, v in per.items():
        out[names[d]].append(v)
    return out


def calibration(per_kernel) -> tuple[str, float]:
    """Factor that turns the counter of the calibration copy into its known size."""
    cands = [(n, v) for n, v in per_kernel.items() if COPY_PATTERN.search(n) and "srat::" not in n]
    if len(cands) != 1:
        raise SystemExit(f"expected one copy kernel in the counter file, found {[n for n, _ in cands]}")
    name, vals = cands[0]
    kib = sorted(vals)[len(vals) // 2]
    return name, COPY_BYTES / (kib * 1024.0)


def cmd_stats(a):
    rows = stats_table(a.csv)
    out = a.out or os.path.join(ROOT, "profiles", f"kernels_{a.workload}.md")
    lines = [f"# Kernel durations: {a.workload}", "",
             "rocprofv3 kernel-trace statistics. Command, from the repository root (TMPDIR=/tmp):", "",
             "```", a.command, "```", "",
             "| kernel | calls | mean us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in rows:
        lines.append(f"| {pretty_name(name)} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f}% |")
    if a.note:
        lines += ["", a.note]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def cmd_traffic(a):
    fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(a.write, "WRITE_SIZE")
    cn_f, f_fac = calibration(fetch)
    cn_w, w_fac = calibration(write)
    lines = [f"# HBM traffic per launch: {a.workload}", "",
             "rocprofv3 counters, one pass each (KiB per dispatch, summed over the dispatch's rows, "
             "median over dispatches), scaled by the factor that makes a plain device copy of "
             f"{COPY_BYTES} bytes launched in the same run read (FETCH_SIZE) and write (WRITE_SIZE) "
             "exactly that many bytes.", "",
             "```", a.command_fetch, a.command_write, "```", "",
             f"calibration kernel: `{cn_f[:80]}`; FETCH_SIZE factor {f_fac:.4f}, WRITE_SIZE factor {w_fac:.4f}", "",
             "| kernel | dispatches | fetch MB | write MB | total MB |", "|---|---|---|---|---|"]
    for full in sorted(fetch):
        k = short_name(full)
        if k not in KERNEL_SOURCES or full not in write:
            continue
        fv = sorted(fetch[full])[len(fetch[full]) // 2] * 1024.0 * f_fac
        wv = sorted(write[full])[len(write[full]) // 2] * 1024.0 * w_fac
        rec = {"kernel": k, "workload": a.workload, "instance": full,
               "fetch_bytes_per_launch": fv, "write_bytes_per_launch": wv,
               "hbm_bytes_per_launch": fv + wv, "fetch_factor": f_fac, "write_factor": w_fac,
               "dispatches": len(fetch[full]), "source_hash": src_hash(k),
               "commands": [a.command_fetch, a.command_write]}
        with open(os.path.join(ROOT, "profiles", f"traffic_{k}_{a.workload}.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        lines.append(f"| {k} | {len(fetch[full])} | {fv / 1e6:.2f} | {wv / 1e6:.2f} | {(fv + wv) / 1e6:.2f} |")
    out = os.path.join(ROOT, "profiles", f"traffic_{a.workload}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def counter_means(paths):
    """{library trace name: {counter: mean over dispatches}} over several --pmc passes."""
    out = collections.defaultdict(dict)
    for path in paths:
        with open(path) as f:
            counters = {_col(r, "Counter_Name", "Counter-Name") for r in csv.DictReader(f)}
        for c in sorted(counters):
            for full, vals in counter_per_dispatch(path, c).items():
                k = short_name(full)
                if k in KERNEL_SOURCES:
                    out[k][c] = sum(vals) / len(vals)
    return out


COUNTER_NOTE = (
    "Normalisation: kernel cycles = `GRBM_GUI_ACTIVE` / 8 XCDs; MFMA busy = `SQ_VALU_MFMA_BUSY_CYCLES` / "
    "1024 SIMDs; VALU busy = 4 x `SQ_ACTIVE_INST_VALU` / 1024 SIMDs (the SQ counts it in units of 4 cycles); "
    "LDS busy = `SQ_LDS_IDX_ACTIVE` / 256 CUs; all over the kernel cycles. The wave-time shares divide "
    "`SQ_ACTIVE_INST_ANY` (issuing), `SQ_WAIT_INST_ANY` (waiting on an instruction dependency) and "
    "`SQ_WAIT_ANY` (waiting on a memory or LDS counter) by `SQ_WAVE_CYCLES`.")


def cmd_counters(a):
    m = counter_means(a.csv)
    lines = [f"# Issue counters: {a.workload}", "",
             f"rocprofv3 counters, {len(a.csv)} passes (per dispatch, mean over the dispatches of each kernel). "
             "Commands, from the repository root (TMPDIR=/tmp):", "", "```", *a.command, "```", "",
             COUNTER_NOTE, "",
             "| kernel | VALU insts | MFMA insts | LDS insts | kernel cycles | MFMA busy | VALU busy | LDS busy "
             "| LDS bank conflicts / LDS busy | wave issuing | wave waiting on dependency | wave waiting on memory/LDS |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    nan = float("nan")
    for k in KERNEL_SOURCES:
        if k not in m:
            continue
        g = lambda c: m[k].get(c, nan)
        cyc = g("GRBM_GUI_ACTIVE") / 8
        wc = g("SQ_WAVE_CYCLES")
        lds = g("SQ_LDS_IDX_ACTIVE")
        lines.append(
            f"| {k} | {g('SQ_INSTS_VALU'):.0f} | {g('SQ_INSTS_MFMA'):.0f} | {g('SQ_INSTS_LDS'):.0f} | {cyc:.0f} "
            f"| {g('SQ_VALU_MFMA_BUSY_CYCLES') / 1024 / cyc:.0%} | {4 * g('SQ_ACTIVE_INST_VALU') / 1024 / cyc:.0%} "
            f"| {lds / 256 / cyc:.0%} | {g('SQ_LDS_BANK_CONFLICT') / lds if lds else 0:.0%} "
            f"| {g('SQ_ACTIVE_INST_ANY') / wc:.0%} | {g('SQ_WAIT_INST_ANY') / wc:.0%} | {g('SQ_WAIT_ANY') / wc:.0%} |")
    if a.note:
        lines += ["", a.note]
    out = os.path.join(ROOT, "profiles", f"counters_{a.workload}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--out")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True, action="append", help="one counter_collection.csv per pass")
    c.add_argument("--command", required=True, action="append", help="the command of each pass")
    c.add_argument("--workload", required=True)
    c.add_argument("--note", default="")
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
