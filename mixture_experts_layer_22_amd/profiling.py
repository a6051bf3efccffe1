"""Summaries of rocprofv3 output for the profiles/ directory.

    python -m mixture_experts_layer_22_amd.profiling stats  DIR  [--out FILE] [--cmd CMD]
    python -m mixture_experts_layer_22_amd.profiling traffic --kernel NAME
           --copy-fetch DIR --copy-write DIR --fetch DIR --write DIR
           [--copy-bytes N] [--out FILE] [--cmd CMD]
    python -m mixture_experts_layer_22_amd.profiling counters DIR [DIR ...]
           --kernel NAME [--kernel NAME ...] [--out FILE] [--cmd CMD]

`stats` turns a `--kernel-trace --stats` run (CSV output) into a short text
table (with the bench line's phase times, when the run's log is given).  `traffic` turns two counter runs of a workload (FETCH_SIZE, then
WRITE_SIZE) into HBM bytes per launch of one kernel, each scaled by what the
same counter reads for a plain device copy of known size (the copy moves
copy_bytes in and copy_bytes out), and writes a JSON record that bench.py
reports as roofline.traffic while the kernel source is unchanged.
`counters` turns one or more `--pmc` runs into a table of every collected
counter per dispatch of each named kernel (mean over its dispatches), with
MFMA-busy and LDS-conflict ratios derived from them.  The bench's MFMA
ceiling probe (k_mfma_loop, a loop of independent MFMA chains that reaches
about 0.95 of the bf16 peak) runs in the same process, so its own
SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CYCLES ratio calibrates what a busy
MFMA pipe reads on this GPU.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


# source file of each kernel whose traffic is recorded
KERNEL_SOURCES = {
    "k_gemm_dl": "gemm.hip",
    "k_grouped_gemm_bf16": "gemm.hip",
    "k_grouped_gemm_f32": "gemm.hip",
    "k_atomic_h": "combine.hip",
    "k_atomic_combine": "combine.hip",
}


def kernel_source(kernel: str) -> str:
    for k, f in KERNEL_SOURCES.items():
        if kernel.startswith(k):
            return f
    raise KeyError(kernel)


def kernel_source_sha(kernel: str = "k_gemm_dl") -> str:
    with open(os.path.join(HERE, "csrc", kernel_source(kernel)), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _one(pattern):
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def stats_table(run_dir: str, top: int = 20) -> str:
    rows = list(csv.DictReader(open(_one(os.path.join(run_dir, "**", "*kernel_stats.csv")))))
    lines = [f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows[:top]:
        lines.append(f"{r['Name'][:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} "
                     f"{float(r['MinNs'])/1e3:10.2f} {float(r['MaxNs'])/1e3:10.2f} "
                     f"{float(r['Percentage']):6.2f}")
    return "\n".join(lines)


def counter_per_dispatch(run_dir: str, counter: str, kernel_substr: str, reduce: str = "mean"):
    """Mean (or max) over dispatches of kernel `kernel_substr` of the counter
    summed over its instances (FETCH_SIZE / WRITE_SIZE are in KiB)."""
    rows = csv.DictReader(open(_one(os.path.join(run_dir, "**", "*counter_collection.csv"))))
    per = collections.defaultdict(float)
    for r in rows:
        if r["Counter_Name"] != counter or kernel_substr not in r["Kernel_Name"]:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for kernel {kernel_substr!r} in {run_dir}")
    vals = list(per.values())
    if reduce == "max":
        return max(vals), len(vals)
    return sum(vals) / len(vals), len(vals)


def traffic_record(kernel, copy_fetch, copy_write, fetch, write, copy_bytes, copy_kernel="copy"):
    # the copy run also moves small buffers; the calibration copy is the largest
    cf, _ = counter_per_dispatch(copy_fetch, "FETCH_SIZE", copy_kernel, "max")
    cw, _ = counter_per_dispatch(copy_write, "WRITE_SIZE", copy_kernel, "max")
    f, nf = counter_per_dispatch(fetch, "FETCH_SIZE", kernel)
    w, nw = counter_per_dispatch(write, "WRITE_SIZE", kernel)
    fetch_scale = copy_bytes / (cf * 1024.0)
    write_scale = copy_bytes / (cw * 1024.0)
    # the calibration run also streams copy_bytes once through plain loads
    # and once through direct-to-LDS loads: their FETCH_SIZE shows whether
    # the copy's factor holds for both load kinds
    reads = {}
    for k in ("k_stream_read(", "k_stream_read_lds"):
        try:
            reads[k.rstrip("(")] = counter_per_dispatch(copy_fetch, "FETCH_SIZE", k, "max")[0]
        except (ValueError, FileNotFoundError):
            pass
    return {
        "kernel": kernel,
        "fetch_bytes": f * 1024.0 * fetch_scale,
        "write_bytes": w * 1024.0 * write_scale,
        "bytes": f * 1024.0 * fetch_scale + w * 1024.0 * write_scale,
        "fetch_kib_raw": f, "write_kib_raw": w,
        "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": copy_bytes,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "calibration_stream_reads_fetch_kib": reads,
        "dispatches": [nf, nw],
        "source": kernel_source(kernel),
        "source_sha256": kernel_source_sha(kernel),
    }


def counters_by_kernel(run_dirs, kernels):
    """{kernel: {counter: mean per dispatch}} over the runs' counter CSVs."""
    out = {k: {} for k in kernels}
    for d in run_dirs:
        rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
        names = sorted({r["Counter_Name"] for r in rows})
        for k in kernels:
            for c in names:
                try:
                    v, n = counter_per_dispatch(d, c, k)
                except ValueError:
                    continue
                out[k][c] = v
                out[k].setdefault("_dispatches", n)
    return out


def counters_table(run_dirs, kernels, probe="k_mfma_loop"):
    data = counters_by_kernel(run_dirs, kernels + [probe])
    names = sorted({c for k in data for c in data[k] if not c.startswith("_")})
    lines = ["per dispatch, mean over dispatches (counters summed over their instances)", ""]
    lines.append(f"{'counter':34s} " + " ".join(f"{k[:22]:>24s}" for k in kernels + [probe]))
    for c in names:
        lines.append(f"{c:34s} " + " ".join(
            f"{data[k].get(c, float('nan')):24.4g}" for k in kernels + [probe]))

    def ratio(k, a, b):
        v = data[k]
        return v[a] / v[b] if a in v and b in v and v[b] else None

    p_busy = ratio(probe, "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES")
    lines.append("")
    for k in kernels:
        r = ratio(k, "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES")
        if r is not None:
            rel = f", {r / p_busy:.3f} of the MFMA probe's" if p_busy else ""
            lines.append(f"{k}: MFMA busy / SQ busy = {r:.4f}{rel}")
        lc = ratio(k, "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE") or \
            ratio(k, "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES")
        if lc is not None:
            lines.append(f"{k}: LDS bank-conflict cycles per LDS-active (or SQ-busy) cycle = {lc:.4f}")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in data[k]:
            lines.append(f"{k}: bf16 MFMA FLOPs issued (MOPS x 512) = "
                         f"{data[k]['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4g}")
    if p_busy:
        lines.append(f"{probe}: MFMA busy / SQ busy = {p_busy:.4f}")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--out")
    s.add_argument("--cmd", default="")
    s.add_argument("--log", help="the profiled bench run's output (for its phase times)")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", action="append", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, default=1 << 30)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--out")
    t.add_argument("--cmd", default="")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--out")
    c.add_argument("--cmd", default="")
    a = ap.parse_args(argv)
    if a.cmd_name == "stats":
        text = stats_table(a.dir)
        if a.log:
            for line in open(a.log):
                if line.startswith("{") and '"phases_us"' in line:
                    rec = json.loads(line)
                    ph = ", ".join(f"{k} {v:.1f}" for k, v in rec["phases_us"].items())
                    text += (f"\n\nbench line of the same run: {rec['ms_per_step'] * 1e3:.1f} us per step; "
                             f"phases (us, HIP events): {ph}")
        if a.cmd:
            text = f"command: {a.cmd}\n\n{text}\n"
    elif a.cmd_name == "counters":
        text = counters_table(a.dirs, a.kernel)
        if a.cmd:
            text = f"command: {a.cmd}\n\n{text}\n"
    else:
        recs = [traffic_record(k, a.copy_fetch, a.copy_write, a.fetch, a.write, a.copy_bytes,
                               a.copy_kernel) for k in a.kernel]
        out = {"records": recs}
        if a.cmd:
            out["command"] = a.cmd
        text = json.dumps(out, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + ("\n" if not text.endswith("\n") else ""))
    print(text)


if __name__ == "__main__":
    main(sys.argv[1:])
