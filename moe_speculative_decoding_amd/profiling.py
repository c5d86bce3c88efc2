"""Summaries of rocprofv3 output for the verify-pass kernels (host-side text tools).

    python -m moe_speculative_decoding_amd.profiling traffic FETCH_DIR WRITE_DIR MANIFEST
        HBM traffic per deduplicating call from two `rocprofv3 --pmc FETCH_SIZE`
        and `--pmc WRITE_SIZE` runs of `bench.py --counters MANIFEST`.  Each counter is
        scaled by what it reads for a plain 1 GiB device copy in the same run (the
        calibration factor = copy bytes / counted bytes).

    python -m moe_speculative_decoding_amd.profiling traffic FETCH_DIR WRITE_DIR MANIFEST --out JSON
        the same, written with the sha256 of the kernel sources it was taken with

    python -m moe_speculative_decoding_amd.profiling stats TRACE_DIR
        kernel-duration table from a `rocprofv3 --kernel-trace --stats` run.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def kernel_source_hash() -> str:
    """sha256 over every kernel source (name and contents): a counter summary
    is valid only for the sources it was taken with."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under %s" % d)
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def per_dispatch(d: str, counter: str):
    """[(dispatch_id, kernel name, value in bytes)] in dispatch order (counter in KiB)."""
    acc = defaultdict(float)
    names = {}
    for r in _counter_rows(d):
        if r.get("Counter_Name") != counter:
            continue
        k = int(r["Dispatch_Id"])
        acc[k] += float(r["Counter_Value"]) * 1024.0
        names[k] = r["Kernel_Name"]
    return [(k, names[k], acc[k]) for k in sorted(acc)]


def traffic(fetch_dir: str, write_dir: str, manifest_path: str) -> dict:
    with open(manifest_path) as fh:
        man = json.load(fh)
    out = {}
    for label, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = per_dispatch(d, counter)
        # the counted block is the last per_op * ops dispatches of the counted
        # kernel; the three calibration copies are the last non-library
        # dispatches before it
        kname, k = man.get("kernel", "ffn_stream_kernel"), man.get("per_op", 2)
        ffn_idx = [i for i, (_, n, _) in enumerate(rows) if kname in n]
        need = k * len(man["ops"])
        if len(ffn_idx) < need:
            raise ValueError("expected %d %s dispatches, found %d" % (need, kname, len(ffn_idx)))
        first = ffn_idx[-need]
        ffn = [(rows[i][1], rows[i][2]) for i in ffn_idx[-need:]]
        others = [v for (_, n, v) in rows[:first] if "moe::" not in n]
        copies = others[-man["copies"]:]
        # a copy reads copy_bytes and writes copy_bytes
        factor = man["copy_bytes"] / (sum(copies) / len(copies)) if copies else float("nan")
        per_op = [factor * sum(v for _, v in ffn[k * i:k * (i + 1)]) for i in range(len(man["ops"]))]
        out[label] = {"factor": factor, "per_op": per_op, "copies_counted": copies}
    ops = man["ops"]
    by_n = defaultdict(lambda: [0.0, 0.0, 0.0, 0])
    for i, op in enumerate(ops):
        t = by_n[op["n"]]
        t[0] += out["fetch"]["per_op"][i]
        t[1] += out["write"]["per_op"][i]
        t[2] += op["union_bytes"]
        t[3] += 1
    summary = {
        "fetch_factor": out["fetch"]["factor"], "write_factor": out["write"]["factor"],
        "per_n": {str(n): {"fetch_bytes_per_call": v[0] / v[3], "write_bytes_per_call": v[1] / v[3],
                           "union_bytes_per_call": v[2] / v[3], "fetch_over_union": v[0] / v[2]}
                  for n, v in sorted(by_n.items())},
    }
    tot_f = sum(out["fetch"]["per_op"])
    tot_w = sum(out["write"]["per_op"])
    tot_u = sum(op["union_bytes"] for op in ops)
    summary["traffic_bytes_per_call"] = (tot_f + tot_w) / len(ops)
    summary["union_bytes_per_call"] = tot_u / len(ops)
    summary["fetch_over_union"] = tot_f / tot_u
    return summary


def stats(trace_dir: str) -> str:
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    lines = ["| kernel | calls | avg µs | min µs | max µs | % time |", "|---|---|---|---|---|---|"]
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if "moe::" not in r["Name"]:
                    continue
                lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.2f |" % (
                    r["Name"].split("(")[0].replace("void ", ""), r["Calls"],
                    float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(lines)


def main(argv):
    if len(argv) >= 4 and argv[0] == "traffic":
        rec = traffic(argv[1], argv[2], argv[3])
        if len(argv) >= 6 and argv[4] == "--out":
            rec["kernel_source_sha256"] = kernel_source_hash()
            with open(argv[5], "w") as fh:
                json.dump(rec, fh, indent=1)
        print(json.dumps(rec, indent=1))
    elif len(argv) >= 2 and argv[0] == "stats":
        print(stats(argv[1]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
