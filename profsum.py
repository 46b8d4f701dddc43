"""Summaries of rocprofv3 output for the committed profiles (kernel times, HBM traffic).

  python profsum.py stats RUN_kernel_stats.csv OUT.txt --command "..."
      per-kernel call count and duration table of a ``--kernel-trace --stats`` run

  python profsum.py traffic --kernel K --workload W --source FILE[,FILE...]
         --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv --copy-mib N
         --out OUT.json [--command "..."]
      HBM bytes per launch of kernel K from two ``--pmc`` runs (FETCH_SIZE, then WRITE_SIZE;
      KiB per dispatch), each scaled by what the same counter reads for a device copy of N
      MiB (which reads and writes exactly N MiB).  The JSON records the SHA-256 of the
      kernel's source files (concatenated in the order given) so that a reader can tell
      whether the kernel changed since.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import statistics

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bit_kv_cache_compress_amd", "csrc")


def short_name(name: str) -> str:
    """Kernel name without namespaces and parameter lists, template arguments kept."""
    n = name.strip('"')
    n = re.sub(r"^void ", "", n)
    n = n.replace("kvc::(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in n:  # drop the parameter list, keep <...>
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out)[:90]


def stats(csv_path: str, out_path: str, command: str) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# rocprofv3 kernel statistics", f"command: {command}", "",
             f"{'kernel':60s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s} {'% time':>7s}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{short_name(r['Name']):60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{100 * float(r['TotalDurationNs']) / total:7.2f}")
    open(out_path, "w").write("\n".join(lines) + "\n")


def per_dispatch(csv_path: str, counter: str, kernel: str) -> list:
    """Counter value of every dispatch whose short kernel name starts with ``kernel``."""
    vals = collections.defaultdict(float)
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter or not short_name(r["Kernel_Name"]).startswith(kernel):
            continue
        vals[r.get("Dispatch_Id", r.get("Correlation_Id", len(vals)))] += float(r["Counter_Value"])
    return list(vals.values())


def traffic(a) -> dict:
    fetch = per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write = per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cfetch = per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cwrite = per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    if not (fetch and write and cfetch and cwrite):
        raise SystemExit(f"missing dispatches: fetch {len(fetch)} write {len(write)} copy {len(cfetch)}/{len(cwrite)}")
    kib = a.copy_mib * 1024.0
    fs, ws = kib / statistics.median(cfetch), kib / statistics.median(cwrite)
    f_kib, w_kib = statistics.mean(fetch), statistics.mean(write)
    # one file, or several (the kernel's file and the headers it includes), hashed in order
    srcs = a.source.split(",")
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    rec = {
        "kernel": a.kernel, "workload": a.workload, "source": srcs[0] if len(srcs) == 1 else srcs,
        "source_sha256": h.hexdigest(),
        "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
        "dispatches": [len(fetch), len(write)],
        "copy_calibration": {"mib": a.copy_mib, "kernel": a.copy_kernel,
                             "fetch_kib": statistics.median(cfetch), "write_kib": statistics.median(cwrite),
                             "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)},
        "bytes_per_launch": int(round((f_kib * fs + w_kib * ws) * 1024)),
        "command": a.command,
    }
    json.dump(rec, open(a.out, "w"), indent=1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    for k in ("kernel", "workload", "source", "fetch", "write", "copy_fetch", "copy_write", "out"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-mib", type=float, required=True)
    t.add_argument("--copy-kernel", default="__amd_rocclr_copyBuffer")
    t.add_argument("--command", default="")
    a = ap.parse_args()
    if a.cmd == "stats":
        stats(a.csv, a.out, a.command)
    else:
        print(json.dumps(traffic(a)))


if __name__ == "__main__":
    main()
