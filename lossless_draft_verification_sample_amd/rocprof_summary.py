"""Summaries of rocprofv3 output for the profiles/ folder (measurement tooling).

    python -m lossless_draft_verification_sample_amd.rocprof_summary stats DIR OUT.md CMD...
        kernel-trace --stats run (CSV) -> a short Markdown table per kernel
    python -m lossless_draft_verification_sample_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR
        KERNEL WORKLOAD CALIB_BYTES OUT.json
        two --pmc runs (FETCH_SIZE, then WRITE_SIZE, CSV) of the same command,
        which also copied CALIB_BYTES with one plain device copy -> HBM bytes
        per launch of KERNEL, each counter scaled by what it read for the copy

Counter values are KiB per dispatch. The copy calibration turns them into
bytes: factor = CALIB_BYTES / (counter KiB of the copy * 1024), taken
separately for FETCH_SIZE and WRITE_SIZE. The record carries the digest of
the kernel sources it was measured on; bench.py reports it only while the
sources are unchanged.
"""

import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_draft_verification_sample_amd", "csrc")


def source_digest():
    """Digest of the verification path's kernel sources, the files directly in
    csrc/ (the same one bench.py checks; the calibration kernel in csrc/calib/
    is not part of it)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if not os.path.isfile(os.path.join(CSRC, f)):
            continue
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def _one(pattern):
    hits = glob.glob(pattern, recursive=True)
    if len(hits) != 1:
        raise SystemExit(f"expected one file for {pattern}, found {hits}")
    return hits[0]


def short_name(name):
    """'void sv::row_stats_kernel<unsigned short>(sv::RowStatsArgs)' -> 'row_stats_kernel<unsigned short>'"""
    n = name.split("(")[0]
    n = n.replace("void ", "").replace("sv::", "")
    return n


def stats(run_dir, out_path, command, tail=200):
    path = _one(os.path.join(run_dir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    lines = [
        "# rocprofv3 kernel statistics",
        "",
        "Command (from the repository root on one MI355X):",
        "",
        "```",
        " ".join(command),
        "```",
        "",
        "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
        "|---|---:|---:|---:|---:|---:|",
    ]
    for r in rows:
        lines.append(
            f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
            f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
            f"{float(r['Percentage']):.1f}% |")
    # steady state: the last `tail` dispatches of each kernel (the GPU's first
    # ~150 calls run at lower clocks)
    trace = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    if trace:
        per = {}
        for r in csv.DictReader(open(trace[0])):
            per.setdefault(short_name(r["Kernel_Name"]), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        lines += ["", f"Steady state, last {tail} dispatches of each kernel (from the kernel trace):", "",
                  "| kernel | dispatches | average (us) | median (us) |", "|---|---:|---:|---:|"]
        for name, v in per.items():
            d = [x[1] for x in sorted(v)][-tail:]
            lines.append(f"| {name} | {len(d)} | {statistics.mean(d) / 1e3:.1f} | "
                         f"{statistics.median(d) / 1e3:.1f} |")
    lines += ["", f"Kernel sources digest: `{source_digest()}`", ""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def _counter_rows(run_dir):
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    return list(csv.DictReader(open(path)))


def _per_kernel(rows, key):
    vals = [float(r["Counter_Value"]) for r in rows if key(r)]
    if not vals:
        raise SystemExit("no dispatch matched")
    return vals


def traffic(fetch_dir, write_dir, kernel, workload, calib_bytes, out_path):
    calib_bytes = int(calib_bytes)
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == counter]
        # the calibration copy is the largest plain copy dispatch of the run
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        kib = max(float(r["Counter_Value"]) for r in copies)
        factor = calib_bytes / (kib * 1024.0)
        kv = _per_kernel(rows, lambda r: kernel in r["Kernel_Name"])
        out[counter] = {"kib_per_dispatch_median": statistics.median(kv), "dispatches": len(kv),
                        "calibration_copy_kib": kib, "scale": factor,
                        "bytes_per_launch": statistics.median(kv) * 1024.0 * factor}
    rec = {}
    if os.path.exists(out_path):
        rec = json.load(open(out_path))
    rec[f"{kernel}/{workload}"] = {
        "source_digest": source_digest(),
        "read_bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"],
        "write_bytes_per_launch": out["WRITE_SIZE"]["bytes_per_launch"],
        "bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"],
        "counters": out,
    }
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec[f"{kernel}/{workload}"], indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 4 and sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4:])
    elif len(sys.argv) == 8 and sys.argv[1] == "traffic":
        traffic(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
