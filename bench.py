"""Benchmark of the MoE expert operation of a speculative-decoding verify pass on one MI355X.

Workload (default): the OLMoE-shaped layer (E=64, K=8, d=2048, f=1024, bf16
weights and tokens, fp32 accumulation), Markov-reuse routing with p = 0.5,
pass sizes n = 1, 2, 4, 8, over `--layers` distinct layers of weights (each
layer its own 805 MB of experts, so consecutive operations stream different
weights, as a verify pass through a model does; 8 layers are 6.4 GB, far
beyond the 256 MB Infinity Cache).

A step is one verify operation (route -> union -> deduplicating expert FFN
-> combine) for every (n, layer) pair, captured once in a HIP graph and
replayed.  `value` is union bytes streamed per step over the step time
(effective HBM GB/s on union bytes, the deduplicating kernel's bandwidth
definition of the expert-bytes page, Fig. 2).

Per pass size, the expert FFN alone (deduplicating and per-slot) is timed
the same way: a graph holding that n's calls for every layer, replayed, with
HIP events on the stream the kernels run on around the replays.  From these
come u(n), beta_dedup(n) on union bytes, beta_slot(n) on requested bytes,
r(n) (Table 1 of the expert-bytes page), the bytes/bandwidth + fixed-time
fit and the roofline object.  `--cold` adds per-operation timings after a
read-only 1 GiB scrub that evicts L2 and the Infinity Cache.  The CPU
baseline times the float64 oracle on a bounded sample (one layer, n = 1, 2,
4, 8, one thread).

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
    ap.add_argument("--reps", type=int, default=20, help="graph replays per FFN timing")
    ap.add_argument("--p", type=float, default=0.5, help="Markov reuse probability")
    ap.add_argument("--cold", action="store_true", help="also time operations after a scrub")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the Qwen3-, DeepSeek-V2-Lite- and DeepSeek-V3-shaped points")
    ap.add_argument("--profile-step", action="store_true",
                    help="replay only the one-launch step graph (for a kernel trace whose "
                         "per-template averages are the deduplicating launches at n=1,2,4,8)")
    ap.add_argument("--counters", metavar="MANIFEST",
                    help="counter-collection mode: eager launches of every operation's route+union "
                         "and deduplicating FFN plus three 1 GiB calibration copies; writes the "
                         "launch order to MANIFEST (JSON) and no benchmark line")
    return ap.parse_args()


def measured_traffic():
    """HBM bytes per deduplicating launch (FETCH_SIZE + WRITE_SIZE, calibrated)
    from the committed counter summary, or None once the kernel sources have
    changed since the counters were taken."""
    from moe_speculative_decoding_amd.profiling import kernel_source_hash
    path = os.path.join(ROOT, "profiles", "layer_kernel_olmoe_bf16_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return round(rec["traffic_bytes_per_call"])


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_baseline(cfg, p, budget_s):
    """The oracle as it stands, on one host thread, on one layer at n = 1, 2, 4, 8."""
    import oracle
    from synth import make_case
    from threadpoolctl import threadpool_limits
    cases = []
    for n in (1, 2, 4, 8):  # the step's operations of layer 0
        case = make_case(cfg, n, "markov:%s" % p, seed=0, window=0, layer=0)
        ids, _ = oracle.route_topk(case.logits, cfg.K)
        for e in set(int(v) for v in ids.reshape(-1)):
            case.expert(e)  # generate inputs before the clock starts
        cases.append(case)
    total_bytes, total_s, rounds = 0, 0.0, 0
    with threadpool_limits(limits=1):
        while total_s < budget_s:  # whole rounds of the four operations until the budget is spent
            for case in cases:
                t0 = time.perf_counter()
                r = oracle.verify_op(case, "dedup")
                total_s += time.perf_counter() - t0
                total_bytes += r["union_bytes"]
            rounds += 1
    log("cpu oracle: %d rounds of n=1,2,4,8 in %.1f s" % (rounds, total_s))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(total_bytes / total_s / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "cpu": model,
            "sample": "float64 numpy oracle, dedup mode, one OLMoE-shaped layer, Markov p=%s: "
                      "the operations at n=1,2,4,8 (route+union+FFN+combine incl. weight "
                      "decode), %d rounds, %.1f s on one thread" % (p, rounds, total_s)}


def shape_sweep(dev, reps=10):
    """The one-launch pass on the other layer shapes, deduplicating and per-slot:
    Qwen3-30B-A3B (router logits from AR(1) tokens), DeepSeek-V2-Lite (two shared
    experts, Markov p = 0.5, a 16-node draft tree) and DeepSeek-V3 (fp8 weights with
    128x128 block scales; independent and Markov routing, a 32-node tree).  Each point
    replays a graph of one pass per layer (layers alternate, so no pass finds its
    experts in the Infinity Cache); GB/s on union bytes (dedup) and on requested
    bytes (per-slot).  The OLMoE-shaped layer is also run with the other reuse
    probabilities of its recipe (p = 0, 0.8) and with independent routing."""
    import torch

    from moe_speculative_decoding_amd import _lib as L
    from moe_speculative_decoding_amd.layer import DeviceLayer, VerifyBuffers, to_device, verify_layer
    from synth import make_case
    from synth.configs import DSV2LITE, DSV3, OLMOE, QWEN3
    from synth.gen import device_layer_weights

    stream = torch.cuda.current_stream()
    plan = ((OLMOE, 4, (("markov:0.0", 8, False), ("markov:0.8", 8, False), ("iid", 8, False))),
            (QWEN3, 4, tuple(("logits_ar1", n, False) for n in (1, 2, 4, 8))),
            (DSV2LITE, 4, tuple(("markov:0.5", n, False) for n in (1, 2, 4, 8)) +
             (("markov:0.5", 16, True),)),
            (DSV3, 2, tuple(("iid", n, False) for n in (1, 2, 4, 8)) +
             (("markov:0.5", 8, False), ("markov:0.5", 32, True))))
    out = {}
    for cfg, nl, points in plan:
        layers = []
        for l in range(nl):
            w = device_layer_weights(cfg, seed=0, layer=l, device=dev)
            sh = device_layer_weights(cfg, seed=0, layer=l, device=dev, shared=True) if cfg.S else None
            layers.append(DeviceLayer(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype, cfg.x_dtype,
                                      w, sh))
        for routing, n, tree in points:
            ops = []
            for l in range(nl):
                case = make_case(cfg, n, routing, seed=0, window=l, layer=l, tree=tree)
                ops.append((l, to_device(case.x, dev), to_device(case.logits, dev),
                            VerifyBuffers(layers[l], n, dev)))
            rec = {}
            for mode, name in ((L.MOE_MODE_DEDUP, "dedup"), (L.MOE_MODE_PERSLOT, "perslot")):
                for (l, x, lg, b) in ops:
                    verify_layer(layers[l], b, x, lg, n, mode)
                torch.cuda.synchronize()
                for (_, _, _, b) in ops:
                    if L.moe_get_error(b.ws) != L.MOE_OK:
                        raise RuntimeError("device error word set (%s n=%d)" % (cfg.name, n))
                byt = [b.bytes.cpu().tolist() for (_, _, _, b) in ops]
                g = torch.cuda.CUDAGraph()
                st = torch.cuda.Stream()
                st.wait_stream(stream)
                with torch.cuda.stream(st):
                    with torch.cuda.graph(g, stream=st):
                        for (l, x, lg, b) in ops:
                            verify_layer(layers[l], b, x, lg, n, mode)
                stream.wait_stream(st)
                torch.cuda.synchronize()
                g.replay()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) * 1e-3 / (reps * nl)
                del g
                bytes_ = sum(b[0] for b in byt) / len(byt)
                rec[name] = (t, bytes_)
                if mode == L.MOE_MODE_DEDUP:
                    rec["U"] = sum(int(b.U.item()) for (_, _, _, b) in ops) / len(ops)
                    rec["requested"] = sum(b[1] for b in byt) / len(byt)
            (td, ub), (ts, rb) = rec["dedup"], rec["perslot"]
            key = "%s %s n=%d%s" % (cfg.name, routing, n, " tree" if tree else "")
            out[key] = {"U_mean": round(rec["U"], 2), "u": round(ub / rec["requested"], 4),
                        "union_MB": round(ub / 1e6, 1), "us_dedup": round(1e6 * td, 2),
                        "GBs_dedup_union": round(ub / td / 1e9, 1),
                        "pct_peak_dedup": round(100 * ub / td / 1e9 / PEAK_GBS, 1),
                        "us_perslot": round(1e6 * ts, 2),
                        "GBs_perslot_requested": round(rb / ts / 1e9, 1)}
            log("shape %s: %s" % (key, json.dumps(out[key])))
            del ops
        del layers
        torch.cuda.empty_cache()
    return out


def budget_sweep(dev, reps=10):
    """The one-launch pass with a per-layer expert budget (moe_verify_layer_budget,
    kept gates renormalised) against the same pass without one: time, budgeted union
    bytes, GB/s on them, and what the budget costs in the layer output (relative L2 of
    the budgeted output against the unbudgeted one, and the share of gate mass
    dropped).  OLMoE shape at n = 8 (Markov p = 0.5, 8 layers) and the DeepSeek-V3
    shape with a 32-node draft tree (2 layers)."""
    import torch

    from moe_speculative_decoding_amd import _lib as L
    from moe_speculative_decoding_amd.layer import (DeviceLayer, VerifyBuffers, to_device,
                                                    verify_layer, verify_layer_budget)
    from synth import make_case
    from synth.configs import DSV3, OLMOE
    from synth.gen import device_layer_weights

    stream = torch.cuda.current_stream()
    plan = ((OLMOE, 8, "markov:0.5", 8, False, (8, 16, 24)),
            (DSV3, 2, "markov:0.5", 32, True, (32, 64)))
    out = {}
    for cfg, nl, routing, n, tree, budgets in plan:
        layers = [DeviceLayer(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype, cfg.x_dtype,
                              device_layer_weights(cfg, seed=0, layer=l, device=dev))
                  for l in range(nl)]
        ops = []
        for l in range(nl):
            case = make_case(cfg, n, routing, seed=0, window=l, layer=l, tree=tree)
            ops.append((l, to_device(case.x, dev), to_device(case.logits, dev),
                        VerifyBuffers(layers[l], n, dev)))

        def timed(call):
            for op in ops:
                call(*op)
            torch.cuda.synchronize()
            for (_, _, _, b) in ops:
                if L.moe_get_error(b.ws) != L.MOE_OK:
                    raise RuntimeError("device error word set (%s n=%d)" % (cfg.name, n))
            outs = [b.out[:n].double().cpu() for (_, _, _, b) in ops]
            gates = [b.gates[:n].double().cpu() for (_, _, _, b) in ops]
            byt = sum(b.bytes.cpu().tolist()[0] for (_, _, _, b) in ops) / nl
            g = torch.cuda.CUDAGraph()
            st = torch.cuda.Stream()
            st.wait_stream(stream)
            with torch.cuda.stream(st):
                with torch.cuda.graph(g, stream=st):
                    for op in ops:
                        call(*op)
            stream.wait_stream(st)
            torch.cuda.synchronize()
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / (reps * nl)
            del g
            return t, byt, outs, gates

        t0, b0, ref_out, ref_g = timed(
            lambda l, x, lg, b: verify_layer(layers[l], b, x, lg, n, L.MOE_MODE_DEDUP))
        base = "%s %s n=%d%s" % (cfg.name, routing, n, " tree" if tree else "")
        out[base + " no budget"] = {"union_MB": round(b0 / 1e6, 1), "us": round(1e6 * t0, 2),
                                    "GBs_union": round(b0 / t0 / 1e9, 1)}
        log("budget %s: %s" % (base, json.dumps(out[base + " no budget"])))
        for C in budgets:
            kept_mass = []

            def call(l, x, lg, b, C=C):
                verify_layer_budget(layers[l], b, x, lg, n, C, True)

            t, byt, outs, _ = timed(call)
            # the dropped share of gate mass, from the unbudgeted gates and the kept slots
            for (l, _, _, b) in ops:
                keep = (b.slot_rank[:n * cfg.K].cpu() >= 0).reshape(n, cfg.K).double()
                kept_mass.append(float((ref_g[l] * keep).sum() / ref_g[l].sum()))
            dev_rel = [float(torch.linalg.norm(o - r) / torch.linalg.norm(r))
                       for o, r in zip(outs, ref_out)]
            key = "%s C=%d" % (base, C)
            out[key] = {"union_MB": round(byt / 1e6, 1), "us": round(1e6 * t, 2),
                        "GBs_union": round(byt / t / 1e9, 1),
                        "speedup_vs_no_budget": round(t0 / t, 3),
                        "gate_mass_dropped": round(1.0 - sum(kept_mass) / len(kept_mass), 4),
                        "out_rel_l2_vs_no_budget": round(sum(dev_rel) / len(dev_rel), 4)}
            log("budget %s: %s" % (key, json.dumps(out[key])))
        del ops, layers
        torch.cuda.empty_cache()
    return out


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
    from moe_speculative_decoding_amd.layer import (DeviceLayer, VerifyBuffers, to_device,
                                                    verify_layer, verify_layer_auto, verify_pass)
    from synth import make_case
    from synth.configs import OLMOE
    from synth.gen import device_layer_weights

    cfg = OLMOE
    dev = "cuda:0"
    torch.cuda.set_device(0)
    ns = (1, 2, 4, 8)
    routing = "markov:%s" % args.p
    stream = torch.cuda.current_stream()
    DEDUP, SLOT = L.MOE_MODE_DEDUP, L.MOE_MODE_PERSLOT

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
                        "buf_slot": VerifyBuffers(layers[l], n, dev),
                        "buf_layer": VerifyBuffers(layers[l], n, dev),
                        "buf_layer_slot": VerifyBuffers(layers[l], n, dev)})
    torch.cuda.synchronize()

    # eager pass of both modes, chained and in one launch: byte counts, and
    # the reference for graph replays
    def layer_call(op, mode):
        b = op["buf_layer"] if mode == DEDUP else op["buf_layer_slot"]
        verify_layer(layers[op["layer"]], b, op["x"], op["logits"], op["n"], mode)

    # (profile-step mode: the deduplicating one-launch pass only, so that the
    # kernel trace holds nothing but the launches the step times)
    full = not args.profile_step
    for op in ops:
        if full:
            verify_pass(layers[op["layer"]], op["buf"], op["x"], op["logits"], op["n"], DEDUP)
            verify_pass(layers[op["layer"]], op["buf_slot"], op["x"], op["logits"], op["n"], SLOT)
            layer_call(op, SLOT)
        layer_call(op, DEDUP)
    torch.cuda.synchronize()
    for op in ops:
        bufs = (op["buf"], op["buf_slot"], op["buf_layer"], op["buf_layer_slot"]) if full \
            else (op["buf_layer"],)
        for b in bufs:
            if L.moe_get_error(b.ws) != L.MOE_OK:
                raise RuntimeError("device error word set")
        n = op["n"]
        if full and not (torch.equal(op["buf_layer"].out[:n], op["buf"].out[:n]) and
                         torch.equal(op["buf_layer_slot"].out[:n], op["buf_slot"].out[:n])):
            raise RuntimeError("one-launch and chained passes differ")
        b = op["buf_layer"].bytes.cpu().tolist()
        op["U"] = int(op["buf_layer"].U.item())
        op["union_bytes"], op["requested_bytes"] = int(b[0]), int(b[1])
        op["out_eager"] = op["buf_layer"].out[:op["n"]].clone()
        if full:
            slot = op["buf_slot"].out[:op["n"]]
            rel = float((slot - op["out_eager"]).norm() / op["out_eager"].norm())
            # the two modes sum in different orders (matrix-core blocks vs dot
            # products), so h can round to a neighbouring bf16 value in one mode:
            # a few elements differ by ~2^-8 relative, far inside the 1e-2 bound
            if not rel < 1e-3:
                raise RuntimeError("dedup and per-slot outputs differ (rel %.2e)" % rel)
    step_union_bytes = sum(op["union_bytes"] for op in ops)

    if args.counters:
        # under rocprofv3 --pmc: one dispatch sequence per operation, in order
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        for op in ops:
            layer_call(op, DEDUP)
            torch.cuda.synchronize()
        manifest = {"copy_bytes": src.numel() * 4, "copies": 3,
                    "ops": [{"n": op["n"], "layer": op["layer"], "U": op["U"],
                             "union_bytes": op["union_bytes"],
                             "requested_bytes": op["requested_bytes"]} for op in ops],
                    "kernel": "layer_kernel", "per_op": 1,
                    "sequence": "per op: one layer_kernel (deduplicating mode)"}
        with open(args.counters, "w") as fh:
            json.dump(manifest, fh)
        log("counter mode: %d operations written to %s" % (len(ops), args.counters))
        return

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                fn()
        stream.wait_stream(s)
        torch.cuda.synchronize()
        return g

    def ffn(op, mode, st=None):
        lay = layers[op["layer"]]
        if mode == DEDUP:
            b = op["buf"]
            L.moe_expert_ffn_dedup(lay.shape, lay.weights, op["x"], op["n"], b.U, b.union_ids,
                                   b.offsets, b.perm, b.y_slots, None, b.bytes, b.ws, b.ws_bytes, st)
        else:
            b = op["buf_slot"]
            L.moe_expert_ffn_perslot(lay.shape, lay.weights, op["x"], op["n"], b.ids, b.y_slots,
                                     None, b.bytes, b.ws, b.ws_bytes, st)

    # ---------------------------------------------------------- the step
    log("capturing one step (%d operations, one launch each) in a graph" % len(ops))
    g_step = capture(lambda: [layer_call(op, DEDUP) for op in ops])
    for rep in range(3):  # replays must reproduce the eager results exactly
        for op in ops:
            op["buf_layer"].out.zero_()
        torch.cuda.synchronize()
        g_step.replay()
        torch.cuda.synchronize()
        for op in ops:
            if L.moe_get_error(op["buf_layer"].ws) != L.MOE_OK:
                raise RuntimeError("device error word set in replay %d" % rep)
            if not torch.equal(op["buf_layer"].out[:op["n"]], op["out_eager"]):
                raise RuntimeError("graph replay %d differs from the eager pass" % rep)
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g_step.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_union_bytes / (ms_per_step * 1e-3) / 1e9
    log("step: %.3f ms, %.1f GB/s on union bytes" % (ms_per_step, value))
    if args.profile_step:
        log("profile-step mode: %d replays of %d launches, nothing else timed"
            % (args.steps + args.warmup + 3, len(ops)))
        return

    # -------------------------------------------- FFN alone, per n and mode
    def time_graph(g, calls):
        for _ in range(2):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (args.reps * calls)

    per_n = {}
    for n in ns:
        sel = [op for op in ops if op["n"] == n]
        t = {}
        for mode in (DEDUP, SLOT):
            g = capture(lambda: [ffn(op, mode) for op in sel])
            t[mode] = time_graph(g, len(sel))
            del g
        ub = sum(op["union_bytes"] for op in sel) / len(sel)
        rb = sum(op["requested_bytes"] for op in sel) / len(sel)
        per_n[n] = {"t_dedup": t[DEDUP], "t_slot": t[SLOT], "union_bytes": ub,
                    "requested_bytes": rb, "U": float(np.mean([op["U"] for op in sel]))}

    # whole operation per n (graph of that n's operations): the chain of entry
    # points, and one launch in each mode
    for n in ns:
        sel = [op for op in ops if op["n"] == n]
        g = capture(lambda: [verify_pass(layers[op["layer"]], op["buf"], op["x"], op["logits"],
                                         op["n"], DEDUP) for op in sel])
        per_n[n]["t_op"] = time_graph(g, len(sel))
        del g
        for mode, key in ((DEDUP, "t_layer_dedup"), (SLOT, "t_layer_slot")):
            g = capture(lambda: [layer_call(op, mode) for op in sel])
            per_n[n][key] = time_graph(g, len(sel))
            del g

    # chained step, for comparison with the one-launch step
    g_chain = capture(lambda: [verify_pass(layers[op["layer"]], op["buf"], op["x"], op["logits"],
                                           op["n"], DEDUP) for op in ops])
    ms_chain = time_graph(g_chain, 1) * 1e3
    del g_chain

    # the cost model on the one-launch pass (whole operation in either mode)
    for n in ns:
        per_n[n]["t_dedup_ffn"], per_n[n]["t_slot_ffn"] = per_n[n]["t_dedup"], per_n[n]["t_slot"]
        per_n[n]["t_dedup"], per_n[n]["t_slot"] = per_n[n]["t_layer_dedup"], per_n[n]["t_layer_slot"]
    detail = {}
    for n in ns:
        a = cm.aggregate([per_n[n]])
        detail["n=%d" % n] = {
            "U_mean": round(per_n[n]["U"], 3), "u": round(a["u"], 4),
            "us_layer_dedup": round(1e6 * per_n[n]["t_layer_dedup"], 2),
            "us_layer_perslot": round(1e6 * per_n[n]["t_layer_slot"], 2),
            "us_chain_op_dedup": round(1e6 * per_n[n]["t_op"], 2),
            "us_chain_ffn_dedup": round(1e6 * per_n[n]["t_dedup_ffn"], 2),
            "us_chain_ffn_perslot": round(1e6 * per_n[n]["t_slot_ffn"], 2),
            "GBs_dedup_union": round(a["beta_dedup"] / 1e9, 1),
            "GBs_perslot_requested": round(a["beta_slot"] / 1e9, 1),
            "pct_peak_dedup": round(100 * a["beta_dedup"] / 1e9 / PEAK_GBS, 1),
            "r": round(a["r"], 4), "dedup_faster": cm.dedup_faster(a["u"], a["r"]),
            "saving_us": round(1e6 * a["saving"], 2),
        }
        log("n=%d %s" % (n, json.dumps(detail["n=%d" % n])))
    fit = {}
    for mode, bkey, tkey in (("dedup", "union_bytes", "t_dedup"), ("slot", "requested_bytes", "t_slot")):
        beta, t0_ = cm.fit_bandwidth([per_n[n][bkey] for n in ns], [per_n[n][tkey] for n in ns])
        fit[mode] = {"GBs": round(beta / 1e9, 1), "t0_us": round(t0_ * 1e6, 2)}
    fit["crossover_n"] = cm.crossover(ns, [per_n[n]["t_slot"] - per_n[n]["t_dedup"] for n in ns])
    fit["ms_per_step_chained"] = round(ms_chain, 4)

    # ---- mode dispatch and best draft length (expert-bytes page: Eq. (7),
    # the appendix symbols, Table 2) from the one-launch pass at n = 1..8
    model = {n: {"t_dedup": per_n[n]["t_layer_dedup"], "t_slot": per_n[n]["t_layer_slot"],
                 "union_bytes": per_n[n]["union_bytes"],
                 "requested_bytes": per_n[n]["requested_bytes"]} for n in ns}
    for n in range(1, 9):
        if n in model:
            continue
        sel = []
        for l in range(args.layers):
            case = make_case(cfg, n, routing, seed=0, window=l, layer=l)
            sel.append({"n": n, "layer": l, "x": to_device(case.x, dev),
                        "logits": to_device(case.logits, dev),
                        "buf_layer": VerifyBuffers(layers[l], n, dev),
                        "buf_layer_slot": VerifyBuffers(layers[l], n, dev)})
        for op in sel:
            layer_call(op, DEDUP)
        torch.cuda.synchronize()
        byt = [op["buf_layer"].bytes.cpu().tolist() for op in sel]
        t = {}
        for mode in (DEDUP, SLOT):
            g = capture(lambda: [layer_call(op, mode) for op in sel])
            t[mode] = time_graph(g, len(sel))
            del g
        model[n] = {"t_dedup": t[DEDUP], "t_slot": t[SLOT],
                    "union_bytes": sum(b[0] for b in byt) / len(byt),
                    "requested_bytes": sum(b[1] for b in byt) / len(byt)}
        del sel
    # per-slot re-read fit over n = 1..8 (four points would leave three
    # parameters barely determined)
    b_e = layers[0].expert_bytes()
    rr = cm.fit_reread([model[n]["union_bytes"] / b_e for n in sorted(model)],
                       [n * cfg.K for n in sorted(model)], b_e,
                       [model[n]["t_slot"] for n in sorted(model)])
    fit["slot_reread_cost"] = round(rr["reread_cost"], 3)
    for n in model:
        a = cm.aggregate([model[n]])
        model[n].update(u=a["u"], r=a["r"])
        model[n]["mode"] = "dedup" if cm.dedup_faster(a["u"], a["r"]) else "per-slot"
        model[n]["t_best"] = model[n]["t_dedup"] if model[n]["mode"] == "dedup" else model[n]["t_slot"]
    # the step with the mode chosen on the device per pass from each n's measured r
    mode_out = torch.zeros(len(ops), dtype=torch.int32, device=dev)

    def auto_call(i, op):
        verify_layer_auto(layers[op["layer"]], op["buf_layer"], op["x"], op["logits"], op["n"],
                          model[op["n"]]["r"], mode_out[i:i + 1])

    g_auto = capture(lambda: [auto_call(i, op) for i, op in enumerate(ops)])
    ms_auto = time_graph(g_auto, 1) * 1e3
    del g_auto
    picked = mode_out.cpu().tolist()
    V = [model[k + 1]["t_best"] for k in range(8)]  # V(k) = tau(k + 1)
    steps = cm.step_points(V)
    dispatch = {
        "rule": "dedup iff u(n) < r(n), decided on the device from each pass's union",
        "ms_per_step_auto": round(ms_auto, 4),
        "dedup_passes": sum(1 for m in picked if m == DEDUP), "passes": len(picked),
        "per_n": {"n=%d" % n: {"u": round(model[n]["u"], 4), "r": round(model[n]["r"], 4),
                               "mode": model[n]["mode"],
                               "us_dedup": round(1e6 * model[n]["t_dedup"], 2),
                               "us_perslot": round(1e6 * model[n]["t_slot"], 2)}
                  for n in sorted(model)},
    }
    draft = {
        "V_us": [round(1e6 * v, 2) for v in V],
        "a0": round(cm.a0(V), 4),
        "step_points": [[round(a, 4), k] for a, k in steps],
        "k_star": {"a=%.1f" % a: cm.best_draft_length(V, a) for a in (0.3, 0.5, 0.7, 0.8, 0.9)},
        "reading": "V(k) = time of one MoE layer op at n = k+1 in the mode Eq. (7) picks; "
                   "geometric acceptance, T_a(k) = sum_{j<=k} a^j / V(k)",
    }
    log("dispatch: %s" % json.dumps(dispatch))
    log("draft length: %s" % json.dumps(draft))

    # ---- draft-tree selection ahead of the verify pass: EVICT truncation
    # (cost table = the measured per-op times above) and EcoSpec selection
    from synth.gen import draft_tree, expert_bitsets, predicted_sets
    sel_ws = torch.zeros(256, dtype=torch.uint8, device=dev)
    selection = {}
    for N in (32, 64, 1024):
        parent, q = draft_tree(N, 0)
        k = np.arange(1, N + 1)
        cost = np.interp(k + 1, np.arange(1, 9), [1e6 * model[n]["t_best"] for n in range(1, 9)])
        d_par = torch.from_numpy(parent).to(dev)
        d_q = torch.from_numpy(q).to(dev)
        d_c = torch.from_numpy(cost.astype(np.float32)).to(dev)
        order = torch.empty(N, dtype=torch.int32, device=dev)
        kb = torch.empty(1, dtype=torch.int32, device=dev)
        g = capture(lambda: [L.moe_evict_select(d_par, d_q, d_c, N, order, None, None, kb, sel_ws,
                                                256) for _ in range(8)])
        selection["evict_N%d_us" % N] = round(1e6 * time_graph(g, 8), 2)
        del g
    for N, nl, ne, kk, gamma in ((14, 16, 64, 8, 4), (64, 48, 128, 8, 16)):
        parent, q = draft_tree(N, 1)
        bits = expert_bitsets(predicted_sets(N, nl, ne, kk, 1, parent), nl, ne)
        d_par = torch.from_numpy(parent).to(dev)
        d_q = torch.from_numpy(q).to(dev)
        d_pred = torch.from_numpy(bits.view(np.int64)).to(dev)
        selv = torch.empty(gamma, dtype=torch.int32, device=dev)
        g = capture(lambda: [L.moe_ecospec_select(d_par, d_q, d_pred, None, N, bits.shape[1], gamma,
                                                  0.1, selv, None, sel_ws, 256)
                             for _ in range(8)])
        selection["ecospec_N%d_L%d_E%d_g%d_us" % (N, nl, ne, gamma)] = round(1e6 * time_graph(g, 8), 2)
        del g
    # offline Bellman draft-length policy over a reference sequence
    from synth.gen import reference_sequence_inputs
    for N, Lmax in ((2048, 8), (2048, 12)):
        qv, cv = reference_sequence_inputs(N, Lmax, 0)
        d_q = torch.from_numpy(qv).to(dev)
        d_c = torch.from_numpy(cv).to(dev)
        dpv = torch.empty(N + 1, dtype=torch.float64, device=dev)
        kbv = torch.empty(N, dtype=torch.int32, device=dev)
        g = capture(lambda: [L.moe_bellman_policy(d_q, d_c, N, Lmax, dpv, kbv, sel_ws, 256)])
        t = time_graph(g, 1)
        del g
        selection["bellman_N%d_L%d_us" % (N, Lmax)] = round(1e6 * t, 1)
        selection["bellman_N%d_L%d_mean_k" % (N, Lmax)] = round(float(kbv.double().mean()), 3)
    if L.moe_get_error(sel_ws) != L.MOE_OK:
        raise RuntimeError("selection kernels set the error word")
    log("selection: %s" % json.dumps(selection))

    tot_b = sum(per_n[n]["union_bytes"] for n in ns)
    tot_t = sum(per_n[n]["t_layer_dedup"] for n in ns)
    achieved = tot_b / tot_t / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4), "traffic": measured_traffic(),
                "kernel": "layer_kernel (moe_verify_layer, deduplicating), launches of n=1,2,4,8",
                "bytes_per_launch": "(U + S) * 3*d*f*2 B (union expert bytes), mean %.0f"
                                    % (tot_b / len(ns)),
                "launch_us": {"n=%d" % n: round(1e6 * per_n[n]["t_layer_dedup"], 2) for n in ns}}

    cold = None
    if args.cold:
        scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        rec = []
        for op in ops:
            for mode in (DEDUP, SLOT):
                float(scrub.sum())  # read-only eviction of L2 and the Infinity Cache
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                ffn(op, mode)
                e1.record(stream)
                rec.append((op["n"], mode, e0, e1))
        torch.cuda.synchronize()
        cold = {}
        for n in ns:
            for mode, name in ((DEDUP, "us_ffn_dedup"), (SLOT, "us_ffn_perslot")):
                v = [e0.elapsed_time(e1) * 1e3 for (nn, m, e0, e1) in rec if nn == n and m == mode]
                cold.setdefault("n=%d" % n, {})[name] = round(float(np.median(v)), 2)
        log("cold (event-timed, includes ~6 us of dispatch): %s" % json.dumps(cold))

    shapes = None if args.no_shapes else shape_sweep(dev)
    budget = None if args.no_shapes else budget_sweep(dev)

    cpu = None if args.no_cpu else cpu_baseline(cfg, args.p, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "OLMoE-shaped MoE layer verify op (route, union, dedup SwiGLU "
                               "experts, combine; one launch per op), E=64 K=8 d=2048 f=1024, "
                               "Markov routing p=%s, n=1,2,4,8, %d layers, HIP-graph step"
                               % (args.p, args.layers),
                   "global_batch": sum(ns) * args.layers, "seq_len": 1, "parallelism": "none"},
        "roofline": roofline, "cpu_baseline": cpu, "detail": detail, "fit": fit,
        "dispatch": dispatch, "draft_length": draft, "selection": selection,
        "shapes": shapes,
        "budget": budget,
    }
    if cold is not None:
        line["cold"] = cold
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
