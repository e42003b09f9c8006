"""Summaries of rocprofv3 output for the profiles/ folder, and the reader bench.py uses.

    python -m long_context_sparse_08_amd.profiling stats    --csv <run_kernel_stats.csv> --title T
                                                             --command "<cmd>" --out profiles/<name>.md
    python -m long_context_sparse_08_amd.profiling counters --kernel <substring> --source <csrc file>
        --fetch <dir> --write <dir> --copy-fetch <dir> --copy-write <dir> --copy-bytes <B>
        --commands "<cmd1>" "<cmd2>" ... --out profiles/<name>.md

    python -m long_context_sparse_08_amd.profiling utilization --kernel <substring> --source <csrc file>
        --workload <name> --runs <dir> [<dir> ...] --commands "<cmd1>" ... --out profiles/<name>.md

`utilization` records derived hardware counters of one kernel (rocprofv3's MfmaUtil, LdsUtil,
LDSBankConflict, ...: the mean over its dispatches of each counter found in the --pmc runs),
with the same source hash; `utilization_for` returns them while the source is unchanged.

`counters` turns two --pmc runs of a workload (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch)
into HBM bytes per launch of one kernel, each counter scaled by what it reads for a plain
device-to-device copy of known size (the copy kernel runs in its own two --pmc runs).  The
summary keeps a hash of the kernel's source file; `traffic_for` returns None once that file
has changed, so a stale figure is never reported.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
MARK = "<!-- traffic-json: "


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _short(name: str) -> str:
    n = name.replace("void ", "").replace("csa::(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", n)


def kernel_stats(path: str):
    rows = []
    for r in csv.DictReader(open(path)):
        rows.append((_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]), float(r["TotalDurationNs"])))
    rows.sort(key=lambda x: -x[3])
    return rows


UTIL_MARK = "<!-- util-json: "


def counter_means(run_dir: str, kernel_substr: str) -> dict:
    """{counter: (mean over dispatches, dispatches)} of every counter in the --pmc run for
    kernels whose name contains kernel_substr (each dispatch's instances summed)."""
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = r.get("Kernel_Name", r.get("Kernel-Name", ""))
            if kernel_substr not in name:
                continue
            c = r.get("Counter_Name", r.get("Counter-Name"))
            d = r.get("Dispatch_Id", r.get("Dispatch-Id"))
            per.setdefault(c, {})
            per[c][d] = per[c].get(d, 0.0) + float(r.get("Counter_Value", r.get("Counter-Value", 0)))
    return {c: (sum(v.values()) / len(v), len(v)) for c, v in per.items()}


def counter_mean(run_dir: str, counter: str, kernel_substr: str) -> tuple[float, int]:
    """Mean over dispatches of `counter` (summed over its instances) for kernels whose name
    contains kernel_substr; returns (mean, dispatches)."""
    per_dispatch = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = r.get("Kernel_Name", r.get("Kernel-Name", ""))
            if kernel_substr not in name or r.get("Counter_Name", r.get("Counter-Name")) != counter:
                continue
            d = r.get("Dispatch_Id", r.get("Dispatch-Id"))
            per_dispatch[d] = per_dispatch.get(d, 0.0) + float(r.get("Counter_Value", r.get("Counter-Value", 0)))
    if not per_dispatch:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} under {run_dir}")
    vals = list(per_dispatch.values())
    return sum(vals) / len(vals), len(vals)


def write_stats(a):
    rows = kernel_stats(a.csv)
    lines = [f"# {a.title}", "", "Command (from the repository root, on an MI355X):", "", "```", a.command, "```", "",
             "| kernel | calls | average µs | total µs |", "|---|---:|---:|---:|"]
    for n, c, avg, tot in rows:
        lines.append(f"| `{n}` | {c} | {avg / 1e3:.2f} | {tot / 1e3:.1f} |")
    open(a.out, "w").write("\n".join(lines) + "\n")


def write_counters(a):
    f_k, nf = counter_mean(a.fetch, "FETCH_SIZE", a.kernel)
    w_k, nw = counter_mean(a.write, "WRITE_SIZE", a.kernel)
    f_c, _ = counter_mean(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    w_c, _ = counter_mean(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    kib = a.copy_bytes / 1024.0
    f_scale, w_scale = kib / f_c, kib / w_c           # true KiB per counted KiB
    fetch_b = f_k * f_scale * 1024.0
    write_b = w_k * w_scale * 1024.0
    rec = {"kernel": a.kernel, "source": a.source, "source_sha": source_hash(os.path.join(ROOT, a.source)),
           "workload": a.workload, "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "traffic_bytes": round(fetch_b + write_b), "fetch_kib_raw": f_k, "write_kib_raw": w_k,
           "copy_bytes": a.copy_bytes, "copy_fetch_kib_raw": f_c, "copy_write_kib_raw": w_c,
           "fetch_scale": f_scale, "write_scale": w_scale, "dispatches": [nf, nw]}
    lines = [f"# HBM traffic of `{a.kernel}` — {a.workload}", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over instances) from two rocprofv3 --pmc runs",
             "of the workload, each scaled by the same counter's reading for a plain device-to-device copy",
             f"of {a.copy_bytes} bytes (true KiB / counted KiB).", "",
             "| | counted KiB / dispatch | scale | bytes / launch |", "|---|---:|---:|---:|",
             f"| fetch | {f_k:.1f} | {f_scale:.4f} | {fetch_b:.4g} |",
             f"| write | {w_k:.1f} | {w_scale:.4f} | {write_b:.4g} |",
             f"| copy calibration fetch / write | {f_c:.1f} / {w_c:.1f} | | {a.copy_bytes} |", "",
             f"Source `{a.source}` sha256[:16] = `{rec['source_sha']}` (bench.py reports this traffic only while",
             "the file is unchanged).", "", "Commands (from the repository root, on an MI355X):", "", "```"]
    lines += list(a.commands) + ["```", "", MARK + json.dumps(rec) + " -->"]
    open(a.out, "w").write("\n".join(lines) + "\n")


def write_utilization(a):
    vals = {}
    for d in a.runs:
        for c, (mean, n) in counter_means(d, a.kernel).items():
            vals[c] = (mean, n)
    if not vals:
        raise SystemExit(f"no counters for kernels matching {a.kernel!r} under {a.runs}")
    rec = {"kernel": a.kernel, "source": a.source, "source_sha": source_hash(os.path.join(ROOT, a.source)),
           "workload": a.workload, "counters": {c: round(m, 4) for c, (m, _) in sorted(vals.items())},
           "dispatches": {c: n for c, (_, n) in sorted(vals.items())}}
    lines = [f"# Hardware counters of `{a.kernel}` — {a.workload}", "",
             "Derived counters from rocprofv3 --pmc runs of the workload (mean over the kernel's dispatches).",
             "MfmaUtil: percent of the time the matrix cores are busy; LdsUtil: percent of LDS",
             "bandwidth used; LDSBankConflict: percent of LDS cycles lost to bank conflicts.", "",
             "| counter | mean | dispatches |", "|---|---:|---:|"]
    for c, (m, n) in sorted(vals.items()):
        lines.append(f"| {c} | {m:.2f} | {n} |")
    lines += ["", f"Source `{a.source}` sha256[:16] = `{rec['source_sha']}` (bench.py reports these only while",
              "the file is unchanged).", "", "Commands (from the repository root, on an MI355X):", "", "```"]
    lines += list(a.commands) + ["```", "", UTIL_MARK + json.dumps(rec) + " -->"]
    open(a.out, "w").write("\n".join(lines) + "\n")


def _records(mark: str, profiles_dir: str):
    for f in sorted(glob.glob(os.path.join(profiles_dir, "*.md"))):
        for line in open(f, encoding="utf-8"):
            if line.startswith(mark):
                yield json.loads(line[len(mark):].rsplit(" -->", 1)[0])


def utilization_for(kernel: str, workload: str, profiles_dir: str = os.path.join(ROOT, "profiles")):
    """The counters of a committed utilization summary of `kernel` on `workload`, or None when
    there is none or the kernel's source has changed since they were taken."""
    for rec in _records(UTIL_MARK, profiles_dir):
        if rec.get("kernel") != kernel or rec.get("workload") != workload:
            continue
        src = os.path.join(ROOT, rec["source"])
        if os.path.exists(src) and source_hash(src) == rec["source_sha"]:
            return rec["counters"]
    return None


def traffic_for(kernel: str, workload: str, profiles_dir: str = os.path.join(ROOT, "profiles")):
    """HBM bytes per launch of `kernel` on `workload` from a committed counter summary, or None
    when there is none or the kernel's source has changed since the counters were taken."""
    for f in sorted(glob.glob(os.path.join(profiles_dir, "*.md"))):
        for line in open(f, encoding="utf-8"):
            if not line.startswith(MARK):
                continue
            rec = json.loads(line[len(MARK):].rsplit(" -->", 1)[0])
            if rec.get("kernel") != kernel or rec.get("workload") != workload:
                continue
            src = os.path.join(ROOT, rec["source"])
            if os.path.exists(src) and source_hash(src) == rec["source_sha"]:
                return rec
    return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--kernel", required=True)
    c.add_argument("--source", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-fetch", required=True)
    c.add_argument("--copy-write", required=True)
    c.add_argument("--copy-kernel", default="copyBuffer")
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--commands", nargs="+", required=True)
    c.add_argument("--out", required=True)
    u = sub.add_parser("utilization")
    u.add_argument("--kernel", required=True)
    u.add_argument("--source", required=True)
    u.add_argument("--workload", required=True)
    u.add_argument("--runs", nargs="+", required=True)
    u.add_argument("--commands", nargs="+", required=True)
    u.add_argument("--out", required=True)
    a = ap.parse_args()
    {"stats": write_stats, "counters": write_counters, "utilization": write_utilization}[a.cmd](a)


if __name__ == "__main__":
    main()
