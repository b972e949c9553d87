"""Turns rocprofv3 output into the summaries kept under profiles/.

    python -m hybrid_static_pattern_amd.profiling traffic \
        --fetch <out>/pmc_fetch/run_counter_collection.csv \
        --write <out>/pmc_write/run_counter_collection.csv \
        --copy-mib 256 --command "<the rocprofv3 command lines>" --out profiles/

    python -m hybrid_static_pattern_amd.profiling trace \
        --stats <out>/trace/run_kernel_stats.csv --title "..." --command "..." \
        --out profiles/kernels_<workload>.md

The trace summary is the kernel statistics table of `rocprofv3 --kernel-trace --stats`
(calls, average / min / max microseconds, share of the total), one row per kernel.

FETCH_SIZE and WRITE_SIZE are read per dispatch (KiB) for every libsaf kernel and scaled by
the factor that makes the same counters match a plain elementwise copy of known size (the
bench's --calib-copy-mib torch.neg kernel, which reads and writes copy-mib MiB). Each summary records a
hash of the kernel's sources, so a reader can tell when the kernel has changed since the
counters were taken (bench.py then reports the traffic as unknown).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# kernel (short name) -> source files whose text determines it
KERNEL_SOURCES = {
    "hybrid_fwd_kernel": ["fwd_bf16.hip", "saf_device.h"],
    "dkdv_kernel": ["bwd_bf16.hip", "saf_device.h", "frz_amax.h"],
    "dq_kernel": ["bwd_bf16.hip", "saf_device.h", "frz_amax.h"],
    "bwd_delta_kernel": ["bwd_bf16.hip", "saf_device.h", "frz_amax.h"],
    "frz_half_kernel": ["frz_half.hip", "saf_device.h", "frz_amax.h"],
    "frz_amax_kernel": ["frz_half.hip", "saf_device.h", "frz_amax.h"],
    "var_lse_kernel": ["var_score.hip", "saf_device.h"],
    "var_welford_kernel": ["var_score.hip", "saf_device.h"],
}
# workload each kernel's counters are taken on (part of the summary's file name)
KERNEL_WORKLOAD = {"var_lse_kernel": "calibration_N64_H12_T1024", "var_welford_kernel": "calibration_N64_H12_T1024"}
DEFAULT_WORKLOAD = "1b_T8192_r25"
# bench/prof names -> kernel short names
PROF_TO_KERNEL = {"hybrid_fwd": "hybrid_fwd_kernel", "dkdv": "dkdv_kernel", "dq": "dq_kernel",
                  "bwd_delta": "bwd_delta_kernel", "frz_half": "frz_half_kernel",
                  "frz_amax": "frz_amax_kernel", "var_lse": "var_lse_kernel",
                  "var_welford": "var_welford_kernel"}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(full: str) -> str:
    if "at::native" in full:
        return "torch_copy" if "neg" in full.lower() else "torch_other"
    name = full.split("(")[0] if "(anonymous" not in full.split("<")[0] else full
    for k in KERNEL_SOURCES:
        if k in full:
            return k
    return name.replace("void ", "")


def per_dispatch(path: str, counter: str):
    """Mean counter value per dispatch for each kernel in a rocprofv3 counter CSV."""
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            k = short_name(r["Kernel_Name"])
            tot[k] += float(r["Counter_Value"])
            disp[k].add(r["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


def traffic(fetch_csv: str, write_csv: str, copy_mib: int):
    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    f_scale = copy_kib / fetch["torch_copy"]
    w_scale = copy_kib / write["torch_copy"]
    out = {}
    for k in KERNEL_SOURCES:
        if k in fetch and k in write:
            out[k] = dict(fetch_bytes=fetch[k] * 1024 * f_scale, write_bytes=write[k] * 1024 * w_scale,
                          fetch_kib_raw=fetch[k], write_kib_raw=write[k], fetch_scale=f_scale,
                          write_scale=w_scale, source_hash=source_hash(k))
    return out


def summary_path(outdir: str, kernel: str, workload: str | None = None) -> str:
    wl = workload or KERNEL_WORKLOAD.get(kernel, DEFAULT_WORKLOAD)
    return os.path.join(outdir, f"traffic_{kernel}_{wl}.txt")


def write_summaries(data: dict, outdir: str, command: str, workload: str | None = None,
                    kernels=None) -> None:
    for k, d in data.items():
        if kernels and k not in kernels:
            continue
        with open(summary_path(outdir, k, workload), "w") as f:
            wl = workload or KERNEL_WORKLOAD.get(k, DEFAULT_WORKLOAD)
            f.write(f"# HBM traffic of {k} per launch, workload {wl}\n")
            f.write("# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by the factor that makes the\n")
            f.write("# same counters read a plain device copy of known size correctly.\n")
            f.write(f"# command: {command}\n")
            for key, val in d.items():
                f.write(f"{key}: {val}\n")


def read_summary(kernel: str, outdir: str):
    """The committed traffic summary for `kernel`, or None if absent or taken on other sources."""
    path = summary_path(outdir, kernel)
    if not os.path.exists(path):
        return None
    d = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            key, val = line.split(":", 1)
            d[key.strip()] = val.strip()
    if d.get("source_hash") != source_hash(kernel):
        return None
    return {k: (v if k == "source_hash" else float(v)) for k, v in d.items()}


def pretty_kernel(full: str) -> str:
    """Short, readable kernel name: namespaces and argument lists dropped, template kept."""
    if "at::native" in full:
        return "torch elementwise (setup)"
    name = full.replace("void ", "").replace("saf::(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in name:   # drop the parameter list (the outermost parentheses)
        if ch == "(" and depth == 0 and out and out[-1] != "<":
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


def live_timings(bench_log: str) -> dict:
    """kernels_ms of the JSON line that the traced bench.py printed (its live HIP-event
    averages over the timed steps), or {} when there is none."""
    import json
    d = {}
    with open(bench_log) as f:
        for line in f:
            if line.startswith("{"):
                try:
                    d = json.loads(line).get("kernels_ms", {}) or {}
                except ValueError:
                    pass
    return d


def trace_summary(stats_csv: str, title: str, command: str, bench_log: str | None = None) -> str:
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append((pretty_kernel(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda x: -x[5])
    lines = [f"# Kernel trace: {title}", "", "Command (repository root R on the MI355X box):", "", "```",
             command, "```", "", "rocprofv3 kernel statistics (`run_kernel_stats.csv`):", "",
             "| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in rows:
        lines.append(f"| {name} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f}% |")
    live = live_timings(bench_log) if bench_log else {}
    if live:
        lines += ["", "Live HIP-event averages that the same traced bench.py run printed for its timed steps",
                  "(the trace's averages above also count the warm-up and cold-start calls):", "",
                  "| kernel | average us |", "|---|---|"]
        lines += [f"| {k} | {1e3 * v:.1f} |" for k, v in live.items()]
    return "\n".join(lines) + "\n"


def mfma_summary(runs, command: str, n_simd: int = 1024, peak_clock_ghz: float = 2.4,
                 title: str = "1B-shape layer, B=2, H=16, T=8192, d_h=128, bf16") -> str:
    """MFMA utilisation per kernel from one `rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
    SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE` run per label.
    GRBM_GUI_ACTIVE is summed over the 8 XCDs, so /8 is the shader cycles of the dispatch; the
    MFMA-busy fraction is SQ_VALU_MFMA_BUSY_CYCLES over those cycles times the SIMD count,
    and against the published clock the same busy cycles over duration x 2.4 GHz x SIMDs.
    Executed bf16 FLOPs are SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512."""
    lines = [f"# MFMA utilisation from counters ({title})", "",
             "Command (repository root R on the MI355X box):", "", "```", command, "```", "",
             "Counters are collected per dispatch (the kernels run slower under collection than in",
             "`bench.py`). Clock = GRBM_GUI_ACTIVE / 8 XCDs / duration.", "",
             "| run | kernel | dispatches | ms | clock GHz | MFMA busy (of active cycles) | MFMA busy (of 2.4 GHz) | executed bf16 TFLOP/s |",
             "|---|---|---|---|---|---|---|---|"]
    for label, path in runs:
        cnt = collections.defaultdict(lambda: collections.defaultdict(float))
        dur = collections.defaultdict(dict)
        with open(path) as f:
            for r in csv.DictReader(f):
                k = short_name(r["Kernel_Name"])
                if k not in KERNEL_SOURCES:
                    continue
                cnt[k][r["Counter_Name"]] += float(r["Counter_Value"])
                dur[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        for k in cnt:
            n = len(dur[k])
            t = sum(dur[k].values()) / n
            c = {name: v / n for name, v in cnt[k].items()}
            cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / 8
            busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
            if busy == 0:
                continue
            lines.append(f"| {label} | {k} | {n} | {t * 1e3:.3f} | {cyc / t / 1e9:.2f} | {busy / (cyc * n_simd):.3f} | "
                         f"{busy / (t * peak_clock_ghz * 1e9 * n_simd):.3f} | "
                         f"{c.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0.0) * 512 / t / 1e12:.0f} |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    mf = sub.add_parser("mfma")
    mf.add_argument("--run", action="append", required=True, help="LABEL=path/to/run_counter_collection.csv")
    mf.add_argument("--command", default="")
    mf.add_argument("--out", required=True)
    mf.add_argument("--title", default="1B-shape layer, B=2, H=16, T=8192, d_h=128, bf16")
    tr = sub.add_parser("trace")
    tr.add_argument("--stats", required=True)
    tr.add_argument("--title", required=True)
    tr.add_argument("--command", default="")
    tr.add_argument("--out", required=True)
    tr.add_argument("--bench-log", default=None, help="stdout of the traced bench.py (for its live timings)")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--command", default="")
    t.add_argument("--out", default=os.path.join(os.path.dirname(PKG), "profiles"))
    t.add_argument("--workload", default=None, help="workload name in the summaries' file names")
    t.add_argument("--kernels", default=None, help="comma-separated kernels to write (default: all)")
    a = ap.parse_args()
    if a.cmd == "mfma":
        runs = [tuple(x.rsplit("=", 1)) for x in a.run]
        with open(a.out, "w") as f:
            f.write(mfma_summary(runs, a.command, title=a.title))
        print(f"wrote {a.out}")
        return
    if a.cmd == "trace":
        with open(a.out, "w") as f:
            f.write(trace_summary(a.stats, a.title, a.command, a.bench_log))
        print(f"wrote {a.out}")
        return
    data = traffic(a.fetch, a.write, a.copy_mib)
    write_summaries(data, a.out, a.command, a.workload, a.kernels.split(",") if a.kernels else None)
    for k, d in data.items():
        print(f"{k}: fetch {d['fetch_bytes'] / 1e6:.1f} MB, write {d['write_bytes'] / 1e6:.1f} MB per launch")


if __name__ == "__main__":
    main()
