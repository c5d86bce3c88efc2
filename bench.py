"""Benchmark of the MoE expert operation of a speculative-decoding verify pass on one MI355X.

Workload (default): the OLMoE-shaped layer (E=64, K=8, d=2048, f=1024, bf16
weights and tokens, fp32 accumulation), Markov-reuse routing with p = 0.5,
pass sizes n = 1, 2, 4, 8, over `--layers` distinct layers of weights (each
layer its own 805 MB of experts, so consecutive operations stream different
weights, as a verify pass through a model does).

A step is one verify operation (route -> union -> deduplicating expert FFN
-> combine) for every (n, layer) pair.  The step is captured once in a HIP
graph and replayed; `value` is union bytes streamed per step over the step
time (effective HBM GB/s on union bytes, the deduplicating kernel's
bandwidth definition of the expert-bytes page, Fig. 2).

Per-operation detail is measured separately with a cold cache (a 1 GiB
scrub before every operation, outside the events): the expert FFN of both
modes alone and the whole operation, timed with HIP events on the stream the
kernels run on; r(n), u(n), the bytes/bandwidth + fixed-time fit and the
roofline object come from these.  The CPU baseline times the float64 oracle
on the host on a bounded sample (one layer, n = 1, 2, 4, 8).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--layers 8]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s (union bytes) + µs per MoE verify op at n=1..8; % of peak"
PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--reps", type=int, default=3, help="cold-cache repetitions per operation")
    ap.add_argument("--p", type=float, default=0.5, help="Markov reuse probability")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu", action="store_true")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_baseline(cfg, p, budget_s):
    """The oracle as it stands, on one host thread, on one layer at n = 1, 2, 4, 8."""
    import oracle
    from synth import make_case
    from threadpoolctl import threadpool_limits
    total_bytes, total_s, done = 0, 0.0, []
    with threadpool_limits(limits=1):
        for n in (1, 2, 4, 8):
            case = make_case(cfg, n, "markov:%s" % p, seed=0, window=0, layer=0)
            ids, _ = oracle.route_topk(case.logits, cfg.K)
            for e in set(int(v) for v in ids.reshape(-1)):
                case.expert(e)  # generate inputs before the clock starts
            t0 = time.perf_counter()
            r = oracle.verify_op(case, "dedup")
            dt = time.perf_counter() - t0
            total_bytes += r["union_bytes"]
            total_s += dt
            done.append(n)
            log("cpu oracle n=%d: %.2f s" % (n, dt))
            if total_s > budget_s:
                break
    return {"value": total_bytes / total_s / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "float64 numpy oracle, dedup mode, one OLMoE-shaped layer, Markov p=%s, "
                      "n in %s (route+union+FFN+combine incl. weight decode), one thread"
                      % (p, done)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_speculative_decoding_amd import _lib as L
    from moe_speculative_decoding_amd import costmodel as cm
    from moe_speculative_decoding_amd.layer import DeviceLayer, VerifyBuffers, to_device, verify_pass
    from synth import make_case
    from synth.configs import OLMOE
    from synth.gen import device_layer_weights

    cfg = OLMOE
    dev = "cuda:0"
    torch.cuda.set_device(0)
    ns = (1, 2, 4, 8)
    routing = "markov:%s" % args.p
    stream = torch.cuda.current_stream()

    log("generating %d layers of %s weights on the device" % (args.layers, cfg.name))
    layers = []
    for l in range(args.layers):
        w = device_layer_weights(cfg, seed=0, layer=l, device=dev)
        layers.append(DeviceLayer(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype, cfg.x_dtype, w))
    ops = []
    for n in ns:
        for l in range(args.layers):
            case = make_case(cfg, n, routing, seed=0, window=l, layer=l)
            ops.append({"n": n, "layer": l, "x": to_device(case.x, dev),
                        "logits": to_device(case.logits, dev),
                        "buf": VerifyBuffers(layers[l], n, dev),
                        "buf_slot": VerifyBuffers(layers[l], n, dev)})
    torch.cuda.synchronize()

    # eager pass of both modes: byte counts, and the reference for graph replays
    for op in ops:
        verify_pass(layers[op["layer"]], op["buf"], op["x"], op["logits"], op["n"], L.MOE_MODE_DEDUP)
        verify_pass(layers[op["layer"]], op["buf_slot"], op["x"], op["logits"], op["n"],
                    L.MOE_MODE_PERSLOT)
    torch.cuda.synchronize()
    for op in ops:
        if L.moe_get_error(op["buf"].ws) != L.MOE_OK:
            raise RuntimeError("device error word set")
        b = op["buf"].bytes.cpu().tolist()
        op["U"] = int(op["buf"].U.item())
        op["union_bytes"], op["requested_bytes"] = int(b[0]), int(b[1])
        op["out_eager"] = op["buf"].out[:op["n"]].clone()
        slot = op["buf_slot"].out[:op["n"]]
        rel = float((slot - op["out_eager"]).norm() / op["out_eager"].norm())
        if not rel < 1e-5:
            raise RuntimeError("dedup and per-slot outputs differ (rel %.2e)" % rel)
    step_union_bytes = sum(op["union_bytes"] for op in ops)

    # one step captured in a graph
    log("capturing one step (%d operations) in a graph" % len(ops))
    graph = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(stream)
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(graph, stream=cap_stream):
            for op in ops:
                verify_pass(layers[op["layer"]], op["buf"], op["x"], op["logits"], op["n"],
                            L.MOE_MODE_DEDUP)
    stream.wait_stream(cap_stream)
    torch.cuda.synchronize()
    for rep in range(3):  # replays must reproduce the eager results exactly
        for op in ops:
            op["buf"].out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for op in ops:
            if not torch.equal(op["buf"].out[:op["n"]], op["out_eager"]):
                raise RuntimeError("graph replay %d differs from the eager pass" % rep)

    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_union_bytes / (ms_per_step * 1e-3) / 1e9
    log("graph step: %.3f ms, %.1f GB/s on union bytes" % (ms_per_step, value))

    # cold-cache per-operation timing with events on the kernels' stream
    scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    scrub.zero_()
    rec = []
    for rep in range(args.reps):
        for op in ops:
            lay = layers[op["layer"]]
            for mode, buf in (("dedup", op["buf"]), ("slot", op["buf_slot"])):
                scrub.add_(1.0)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                if mode == "dedup":
                    L.moe_expert_ffn_dedup(lay.shape, lay.weights, op["x"], op["n"], buf.U,
                                           buf.union_ids, buf.offsets, buf.perm, buf.y_slots, None,
                                           buf.bytes, buf.ws, buf.ws_bytes, stream)
                else:
                    L.moe_expert_ffn_perslot(lay.shape, lay.weights, op["x"], op["n"], buf.ids,
                                             buf.y_slots, None, buf.bytes, buf.ws, buf.ws_bytes,
                                             stream)
                e1.record(stream)
                scrub.add_(1.0)
                w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                w0.record(stream)
                verify_pass(lay, buf, op["x"], op["logits"], op["n"],
                            L.MOE_MODE_DEDUP if mode == "dedup" else L.MOE_MODE_PERSLOT, stream)
                w1.record(stream)
                rec.append((op, mode, e0, e1, w0, w1))
    torch.cuda.synchronize()
    for op in ops:
        op.setdefault("t_ffn", {"dedup": [], "slot": []})
        op.setdefault("t_op", {"dedup": [], "slot": []})
    for op, mode, e0, e1, w0, w1 in rec:
        op["t_ffn"][mode].append(e0.elapsed_time(e1) * 1e-3)
        op["t_op"][mode].append(w0.elapsed_time(w1) * 1e-3)

    detail = {}
    fit_rows = {"dedup": ([], []), "slot": ([], [])}
    agg_all = []
    for n in ns:
        sel = [op for op in ops if op["n"] == n]
        rows = []
        for op in sel:
            td = float(np.median(op["t_ffn"]["dedup"]))
            ts = float(np.median(op["t_ffn"]["slot"]))
            rows.append({"union_bytes": op["union_bytes"], "requested_bytes": op["requested_bytes"],
                         "t_dedup": td, "t_slot": ts})
            fit_rows["dedup"][0].append(op["union_bytes"]); fit_rows["dedup"][1].append(td)
            fit_rows["slot"][0].append(op["requested_bytes"]); fit_rows["slot"][1].append(ts)
        agg_all.extend(rows)
        a = cm.aggregate(rows)
        t_op = float(np.mean([np.median(op["t_op"]["dedup"]) for op in sel]))
        detail["n=%d" % n] = {
            "U_mean": float(np.mean([op["U"] for op in sel])),
            "u": round(a["u"], 4),
            "us_ffn_dedup": round(1e6 * float(np.mean([r["t_dedup"] for r in rows])), 2),
            "us_ffn_perslot": round(1e6 * float(np.mean([r["t_slot"] for r in rows])), 2),
            "us_op_dedup": round(1e6 * t_op, 2),
            "GBs_dedup_union": round(a["beta_dedup"] / 1e9, 1),
            "GBs_perslot_requested": round(a["beta_slot"] / 1e9, 1),
            "pct_peak_dedup": round(100 * a["beta_dedup"] / 1e9 / PEAK_GBS, 1),
            "r": round(a["r"], 4),
            "dedup_faster": cm.dedup_faster(a["u"], a["r"]),
        }
        log("n=%d %s" % (n, json.dumps(detail["n=%d" % n])))
    fit = {}
    for mode, (b, t) in fit_rows.items():
        beta, t0_ = cm.fit_bandwidth(b, t)
        fit[mode] = {"GBs": round(beta / 1e9, 1), "t0_us": round(t0_ * 1e6, 2)}
    rr = cm.fit_reread([op["U"] for op in ops], [op["n"] * cfg.K for op in ops],
                       layers[0].expert_bytes(), [r["t_slot"] for r in agg_all])
    fit["slot_reread_cost"] = round(rr["reread_cost"], 3)

    tot_bytes = sum(r["union_bytes"] for r in agg_all)
    tot_t = sum(r["t_dedup"] for r in agg_all)
    achieved = tot_bytes / tot_t / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4), "traffic": None,
                "kernel": "expert FFN, deduplicating (up + down kernels), cold cache",
                "bytes_per_launch": "(U + S) * 3*d*f*2 B"}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, args.p, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "OLMoE-shaped MoE layer verify op (route, union, dedup SwiGLU "
                               "experts, combine), E=64 K=8 d=2048 f=1024, Markov routing "
                               "p=%s, n=1,2,4,8, %d layers, HIP-graph step" % (args.p, args.layers),
                   "global_batch": sum(ns) * args.layers, "seq_len": 1, "parallelism": "none"},
        "roofline": roofline, "cpu_baseline": cpu, "detail": detail, "fit": fit,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
