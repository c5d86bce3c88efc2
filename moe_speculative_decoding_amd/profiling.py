"""Summaries of rocprofv3 output for the verify-pass kernels (host-side text tools).

    python -m moe_speculative_decoding_amd.profiling traffic FETCH_DIR WRITE_DIR MANIFEST
        HBM traffic per one-launch pass (both modes) from two `rocprofv3 --pmc FETCH_SIZE`
        and `--pmc WRITE_SIZE` runs of `bench.py --counters MANIFEST`.  Each counter is
        scaled by what it reads for a plain 1 GiB device copy in the same run (the
        calibration factor = copy bytes / counted bytes).

    python -m moe_speculative_decoding_amd.profiling traffic FETCH_DIR WRITE_DIR MANIFEST --out JSON
        the same, written with the sha256 of the kernel sources it was taken with

    python -m moe_speculative_decoding_amd.profiling stats TRACE_DIR
        kernel-duration table from a `rocprofv3 --kernel-trace --stats` run.

    python -m moe_speculative_decoding_amd.profiling step TRACE_DIR MANIFEST
        mean duration of every operation of the step, from a kernel trace of
        `bench.py --profile-step --step-manifest MANIFEST`.

    python -m moe_speculative_decoding_amd.profiling valu PMC_DIR MANIFEST
        VALUBusy, VALU and MFMA instruction counts per pass from a `--pmc` run of
        `bench.py --counters MANIFEST`.

    python -m moe_speculative_decoding_amd.profiling counters PMC_DIR MANIFEST NAME [NAME ...]
        the mean of each named counter per pass (mode, routing, n) from a `--pmc`
        run of `bench.py --counters MANIFEST` (values as rocprofv3 reports them,
        summed over the counter's instances).
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


def _counted(d: str, counter: str, man: dict):
    """(calibration factor, [bytes of launch i of the manifest]) for one counter run."""
    rows = per_dispatch(d, counter)
    kname = man.get("kernel", "layer_kernel")
    need = len(man["launches"])
    idx = [i for i, (_, n, _) in enumerate(rows) if kname in n]
    if len(idx) < need:
        raise ValueError("expected %d %s dispatches, found %d" % (need, kname, len(idx)))
    first = idx[-need]
    # the three calibration copies are the last dispatches before the counted
    # launches that are not the library's (a copy reads and writes copy_bytes)
    others = [v for (_, n, v) in rows[:first] if "moe::" not in n]
    copies = others[-man["copies"]:]
    factor = man["copy_bytes"] / (sum(copies) / len(copies)) if copies else float("nan")
    return factor, [factor * rows[i][2] for i in idx[-need:]]


def traffic(fetch_dir: str, write_dir: str, manifest_path: str) -> dict:
    """HBM bytes per one-launch pass from a FETCH_SIZE and a WRITE_SIZE run of
    `bench.py --counters`: per mode and (routing, n), against the union bytes
    U*b (both modes) and the requested bytes n*(K+S)*b (per-slot)."""
    with open(manifest_path) as fh:
        man = json.load(fh)
    ff, fetch = _counted(fetch_dir, "FETCH_SIZE", man)
    wf, write = _counted(write_dir, "WRITE_SIZE", man)
    out = {"workload": man.get("workload"), "fetch_factor": ff, "write_factor": wf,
           "expert_bytes": man.get("expert_bytes")}
    for mode in ("dedup", "perslot"):
        sel = [i for i, l in enumerate(man["launches"]) if l["mode"] == mode]
        if not sel:
            continue
        groups = defaultdict(list)
        for i in sel:
            l = man["launches"][i]
            groups["%s n=%d" % (l["routing"], l["n"])].append(i)
        pts = {}
        for key, ii in groups.items():
            f = sum(fetch[i] for i in ii) / len(ii)
            w = sum(write[i] for i in ii) / len(ii)
            ub = sum(man["launches"][i]["union_bytes"] for i in ii) / len(ii)
            rb = sum(man["launches"][i]["requested_bytes"] for i in ii) / len(ii)
            pts[key] = {"fetch_bytes_per_call": f, "write_bytes_per_call": w,
                        "union_bytes_per_call": ub, "requested_bytes_per_call": rb,
                        "fetch_over_union": f / ub, "fetch_over_requested": f / rb}
        tf = sum(fetch[i] for i in sel)
        tw = sum(write[i] for i in sel)
        tu = sum(man["launches"][i]["union_bytes"] for i in sel)
        tr = sum(man["launches"][i]["requested_bytes"] for i in sel)
        out[mode] = {"points": pts, "traffic_bytes_per_call": (tf + tw) / len(sel),
                     "fetch_bytes_per_call": tf / len(sel),
                     "union_bytes_per_call": tu / len(sel), "fetch_over_union": tf / tu,
                     "fetch_over_requested": tf / tr}
    return out


def counter_means(d: str, manifest_path: str, names) -> dict:
    """Mean per pass (mode, routing, n) of each named counter, from a `--pmc`
    run of `bench.py --counters`: the manifest's launches are the run's last
    dispatches of its kernel, in order."""
    with open(manifest_path) as fh:
        man = json.load(fh)
    kname = man.get("kernel", "layer_kernel")
    vals = {}
    for r in _counter_rows(d):
        if kname not in r["Kernel_Name"]:
            continue
        k = int(r["Dispatch_Id"])
        vals.setdefault(k, defaultdict(float))[r["Counter_Name"]] += float(r["Counter_Value"])
    ids = sorted(vals)[-len(man["launches"]):]
    if len(ids) < len(man["launches"]):
        raise ValueError("expected %d %s dispatches, found %d"
                         % (len(man["launches"]), kname, len(ids)))
    groups = defaultdict(list)
    for k, l in zip(ids, man["launches"]):
        groups["%s %s n=%d" % (l["mode"], l["routing"], l["n"])].append(vals[k])
    return {key: {c: sum(v.get(c, 0.0) for v in vs) / len(vs) for c in names}
            for key, vs in groups.items()}


def valu(d: str, manifest_path: str) -> dict:
    """VALU activity per one-launch pass from a `--pmc VALUBusy SQ_INSTS_VALU
    SQ_INSTS_MFMA` run of `bench.py --counters` (VALUBusy: the share of the
    kernel's GPU time in which vector ALU instructions are processed, the
    vendor's derived counter)."""
    return counter_means(d, manifest_path, ("VALUBusy", "SQ_INSTS_VALU", "SQ_INSTS_MFMA"))


def step_stats(trace_dir: str, manifest_path: str) -> dict:
    """Mean duration of each operation of the step from a `--kernel-trace` run
    of `bench.py --profile-step --step-manifest`: the layer_kernel dispatches
    repeat the step's operation order, so dispatch i belongs to operation
    i mod ops; per (routing, n), and the step's union bytes over its summed
    mean durations."""
    with open(manifest_path) as fh:
        man = json.load(fh)
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if "layer_kernel" in r["Kernel_Name"]:
                    rows.append((int(r["Start_Timestamp"]),
                                 int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    ops = man["ops"]
    if len(rows) % len(ops) != 0:
        raise ValueError("%d layer_kernel dispatches for %d operations" % (len(rows), len(ops)))
    reps = len(rows) // len(ops)
    per_op = [0.0] * len(ops)
    for i, (_, dur) in enumerate(rows):
        per_op[i % len(ops)] += dur / reps
    groups = defaultdict(list)
    for i, op in enumerate(ops):
        groups["%s n=%d" % (op["routing"], op["n"])].append(i)
    pts = {key: {"us": sum(per_op[i] for i in ii) / len(ii) / 1e3,
                 "union_bytes": sum(ops[i]["union_bytes"] for i in ii) / len(ii)}
           for key, ii in groups.items()}
    tb = sum(op["union_bytes"] for op in ops)
    tt = sum(per_op) * 1e-9
    return {"replays": reps, "points": pts, "step_kernel_us": sum(per_op) / 1e3,
            "GBs_union": tb / tt / 1e9}


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
    if len(argv) >= 3 and argv[0] == "valu":
        print(json.dumps(valu(argv[1], argv[2]), indent=1))
    elif len(argv) >= 3 and argv[0] == "step":
        print(json.dumps(step_stats(argv[1], argv[2]), indent=1))
    elif len(argv) >= 4 and argv[0] == "traffic":
        rec = traffic(argv[1], argv[2], argv[3])
        if len(argv) >= 6 and argv[4] == "--out":
            rec["kernel_source_sha256"] = kernel_source_hash()
            with open(argv[5], "w") as fh:
                json.dump(rec, fh, indent=1)
        print(json.dumps(rec, indent=1))
    elif len(argv) >= 4 and argv[0] == "counters":
        print(json.dumps(counter_means(argv[1], argv[2], argv[3:]), indent=1))
    elif len(argv) >= 2 and argv[0] == "stats":
        print(stats(argv[1]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
