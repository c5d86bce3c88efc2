"""Benchmark of the MoE expert operation of a speculative-decoding verify pass on one MI355X.

Workload of the headline line: the DeepSeek-V3-shaped layer (E=256 routed
experts, K=8, d=7168, f=2048; fp8 E4M3FN expert weights with one fp32 scale
per 128x128 block, 44.05 MB per expert, 11.3 GB per layer; bf16 tokens), the
largest layer shape of the workloads that fits one GPU.  Pass sizes n = 1..8,
with independent uniform routing and with Markov-reuse routing (p = 0.5),
over `--layers` distinct layers of weights, so consecutive operations stream
different weights as a verify pass through a model does (every pass streams
352 MB or more, beyond the 256 MB Infinity Cache).

A step is one verify operation (route -> union -> deduplicating expert FFN
-> combine, one launch) for every (routing, n, layer) triple, captured once
in a HIP graph and replayed.  `value` is the union bytes the step streams
over the step time: effective HBM GB/s on union bytes, the deduplicating
kernel's bandwidth definition of the expert-bytes page (Fig. 2, Table 1).

Per (routing, n), the one-launch pass in each mode is timed the same way (a
graph of that point's launches, replayed, with HIP events on the launch
stream).  From these come u(n), beta_dedup(n) on union bytes, beta_slot(n)
on requested bytes, r(n) (Table 1 of the expert-bytes page), the
bytes/bandwidth + fixed-time fit, the sign check of Eq. (19), the roofline
object and the mode each pass size gets from Eq. (7).  The OLMoE-shaped bf16
layer (n = 1, 2, 4, 8, Markov p = 0.5, 8 layers) is measured alongside
(`olmoe`), and the other layer shapes in `shapes`.  The CPU baseline times
the float64 oracle on a bounded sample of the headline workload, on one
thread and on every host core.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--layers 4]
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
HEADLINE_ROUTINGS = ("iid", "markov:0.5")
HEADLINE_NS = (1, 2, 3, 4, 5, 6, 7, 8)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=4,
                    help="DeepSeek-V3-shaped layers of weights (11.3 GB each)")
    ap.add_argument("--olmoe-layers", type=int, default=8)
    ap.add_argument("--reps", type=int, default=20, help="graph replays per point timing")
    ap.add_argument("--cpu-experts", type=int, default=64,
                    help="union experts per pass in the CPU baseline's sample (64: the "
                         "whole union of every pass of up to 8 tokens)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the OLMoE, Qwen3, DeepSeek-V2-Lite and tree points and the "
                         "budget and selection sweeps")
    ap.add_argument("--workload", choices=("dsv3", "olmoe", "dsv3tree"), default="dsv3",
                    help="the workload of --profile-step / --counters (dsv3tree: the "
                         "DeepSeek-V3-shaped layer with 32-node draft trees, 2 layers)")
    ap.add_argument("--profile-step", action="store_true",
                    help="replay only the one-launch step graph of --workload (for a kernel "
                         "trace whose layer_kernel dispatches are the step's launches)")
    ap.add_argument("--step-manifest", metavar="PATH",
                    help="with --profile-step: write the step's operation order (routing, n, "
                         "layer, union bytes) to PATH for `profiling step`")
    ap.add_argument("--counters", metavar="MANIFEST",
                    help="counter-collection mode: three 1 GiB calibration copies, then one "
                         "eager one-launch pass per operation of --workload in each mode, a "
                         "synchronisation after each; writes the launch order to MANIFEST "
                         "(JSON) and no benchmark line")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def measured_traffic(workload):
    """HBM bytes per deduplicating launch of the step (FETCH_SIZE + WRITE_SIZE,
    calibrated) from the committed counter summary, or None once the kernel
    sources have changed since the counters were taken."""
    from moe_speculative_decoding_amd.profiling import kernel_source_hash
    path = os.path.join(ROOT, "profiles", "layer_kernel_%s_traffic.json" % workload)
    if not os.path.exists(path):
        return None, None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None, rec
    return round(rec["dedup"]["traffic_bytes_per_call"]), rec


# ------------------------------------------------------------------ helpers
def capture(fn):
    """A HIP graph of everything fn enqueues (captured on a side stream)."""
    import torch
    main = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(main)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    main.wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_graph(g, calls, reps):
    """Seconds per call of a graph of `calls` launches: HIP events on the
    stream the replays run on, around `reps` replays after two untimed ones."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(2):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * calls)


class Runner:
    """Device layers, the operations of a workload and graph timing."""

    def __init__(self, cfg, nlayers, dev):
        import torch

        from moe_speculative_decoding_amd.layer import DeviceLayer
        from synth.gen import device_layer_weights
        self.torch = torch
        self.cfg, self.dev = cfg, dev
        self.layers = []
        for l in range(nlayers):
            w = device_layer_weights(cfg, seed=0, layer=l, device=dev)
            sh = device_layer_weights(cfg, seed=0, layer=l, device=dev, shared=True) if cfg.S else None
            self.layers.append(DeviceLayer(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype,
                                           cfg.x_dtype, w, sh))

    def ops(self, routing, n, tree=False):
        from moe_speculative_decoding_amd.layer import VerifyBuffers, to_device
        from synth import make_case
        out = []
        for l in range(len(self.layers)):
            case = make_case(self.cfg, n, routing, seed=0, window=l, layer=l, tree=tree)
            out.append({"routing": routing, "n": n, "layer": l, "x": to_device(case.x, self.dev),
                        "logits": to_device(case.logits, self.dev),
                        "buf": VerifyBuffers(self.layers[l], n, self.dev),
                        "buf_slot": VerifyBuffers(self.layers[l], n, self.dev)})
        return out

    def call(self, op, mode):
        from moe_speculative_decoding_amd import _lib as L
        from moe_speculative_decoding_amd.layer import verify_layer
        b = op["buf"] if mode == L.MOE_MODE_DEDUP else op["buf_slot"]
        verify_layer(self.layers[op["layer"]], b, op["x"], op["logits"], op["n"], mode)

    def eager(self, ops, chain_check=False, both=True):
        """One eager pass per op (both modes unless both=False): byte counts,
        union sizes and the reference outputs of graph replays; the two modes
        must agree."""
        from moe_speculative_decoding_amd import _lib as L
        from moe_speculative_decoding_amd.layer import VerifyBuffers, verify_pass
        torch = self.torch
        for op in ops:
            self.call(op, L.MOE_MODE_DEDUP)
            if both:
                self.call(op, L.MOE_MODE_PERSLOT)
        torch.cuda.synchronize()
        for op in ops:
            for b in ((op["buf"], op["buf_slot"]) if both else (op["buf"],)):
                if L.moe_get_error(b.ws) != L.MOE_OK:
                    raise RuntimeError("device error word set (%s n=%d)" % (op["routing"], op["n"]))
            n = op["n"]
            bb = op["buf"].bytes.cpu().tolist()
            op["U"] = int(op["buf"].U.item())
            op["union_bytes"], op["requested_bytes"] = int(bb[0]), int(bb[1])
            op["out_eager"] = op["buf"].out[:n].clone()
            if not both:
                continue
            slot = op["buf_slot"].out[:n]
            rel = float((slot - op["out_eager"]).norm() / op["out_eager"].norm())
            # the modes sum in different orders (matrix-core blocks vs dot
            # products), so h can round to a neighbouring bf16 value in one mode
            if not rel < 1e-3:
                raise RuntimeError("dedup and per-slot outputs differ (rel %.2e)" % rel)
        if chain_check:
            # the chain of entry points reproduces the one-launch pass bit for bit
            for op in ops:
                cb = VerifyBuffers(self.layers[op["layer"]], op["n"], self.dev)
                verify_pass(self.layers[op["layer"]], cb, op["x"], op["logits"], op["n"],
                            L.MOE_MODE_DEDUP)
                torch.cuda.synchronize()
                if not torch.equal(cb.out[:op["n"]], op["out_eager"]):
                    raise RuntimeError("one-launch and chained passes differ")
                del cb

    def point(self, ops, reps):
        """The one-launch pass of these ops in both modes: mean time per launch."""
        from moe_speculative_decoding_amd import _lib as L
        t = {}
        for mode in (L.MOE_MODE_DEDUP, L.MOE_MODE_PERSLOT):
            g = capture(lambda: [self.call(op, mode) for op in ops])
            t[mode] = time_graph(g, len(ops), reps)
            del g
        m = len(ops)
        return {"t_dedup": t[L.MOE_MODE_DEDUP], "t_slot": t[L.MOE_MODE_PERSLOT],
                "union_bytes": sum(op["union_bytes"] for op in ops) / m,
                "requested_bytes": sum(op["requested_bytes"] for op in ops) / m,
                "U": sum(op["U"] for op in ops) / m}


def point_record(p):
    from moe_speculative_decoding_amd import costmodel as cm
    a = cm.aggregate([p])
    return {"U_mean": round(p["U"], 2), "u": round(a["u"], 4),
            "union_MB": round(p["union_bytes"] / 1e6, 1),
            "us_dedup": round(1e6 * p["t_dedup"], 2), "us_perslot": round(1e6 * p["t_slot"], 2),
            "GBs_dedup_union": round(a["beta_dedup"] / 1e9, 1),
            "GBs_perslot_requested": round(a["beta_slot"] / 1e9, 1),
            "pct_peak_dedup": round(100 * a["beta_dedup"] / 1e9 / PEAK_GBS, 1),
            "r": round(a["r"], 4), "dedup_faster": cm.dedup_faster(a["u"], a["r"]),
            "saving_us": round(1e6 * a["saving"], 2)}


def fits(points, ns, b_e, K, S):
    """Per mode: tau = bytes / beta + t0 over the pass sizes; the per-slot
    re-read fit; the fit's largest relative residual as the bandwidth error
    eps of Eq. (19), and the sign check at each n."""
    from moe_speculative_decoding_amd import costmodel as cm
    out = {}
    eps = 0.0
    for mode, bkey, tkey in (("dedup", "union_bytes", "t_dedup"), ("slot", "requested_bytes", "t_slot")):
        B = [points[n][bkey] for n in ns]
        T = [points[n][tkey] for n in ns]
        beta, t0 = cm.fit_bandwidth(B, T)
        res = max(abs(t - (b / beta + t0)) / t for b, t in zip(B, T))
        eps = max(eps, res)
        out[mode] = {"GBs": round(beta / 1e9, 1), "t0_us": round(t0 * 1e6, 2),
                     "max_rel_residual": round(res, 4)}
    rr = cm.fit_reread([points[n]["union_bytes"] / b_e - S for n in ns], [n * K for n in ns], b_e,
                       [points[n]["t_slot"] for n in ns])
    out["slot_reread_cost"] = round(rr["reread_cost"], 3)
    out["crossover_n"] = cm.crossover(ns, [points[n]["t_slot"] - points[n]["t_dedup"] for n in ns])
    eq19 = {}
    for n in ns:
        a = cm.aggregate([points[n]])
        eq19["n=%d" % n] = cm.sign_is_robust(a["r"], a["u"], eps)
    out["eq19"] = {"eps": round(eps, 4), "eps_source": "largest relative residual of the two "
                   "bandwidth fits (tau = bytes/beta + t0) over n", "robust": eq19}
    return out


# ------------------------------------------------------------- CPU baseline
def _oracle_pass(cfg, case, mode, threads, n_experts):
    """One verify op of the oracle as it stands: route, union, the FFN of
    `mode` (weight decode included), combine.  On several threads the FFN's
    independent parts go to a pool, one oracle call each: a union expert
    (dedup), a slot (per-slot), the shared experts of the pass (dedup) or of
    a token (per-slot); the rows each call produced are copied into place.
    The deduplicating pass may be capped at its first `n_experts` union
    experts (every slot routed to them).  Returns (seconds, bytes read,
    experts evaluated)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    t0 = time.perf_counter()
    ids, gates = oracle.route_topk(case.logits, cfg.K)
    un = oracle.build_union(ids, cfg.E)
    n = ids.shape[0]
    ffn = (cfg.w_dtype, cfg.x_dtype, cfg.d, cfg.f)
    if mode == "dedup":
        m = min(int(un["U"]), n_experts)
        evals = m + cfg.S

        def part(job):  # union experts [u0, u1) and the first S shared experts
            u0, u1, S = job
            sub = {"U": u1 - u0, "union_ids": un["union_ids"][u0:u1],
                   "offsets": un["offsets"][u0:u1 + 1], "perm": un["perm"]}
            return oracle.ffn_dedup(case.x, ids, sub, case.expert, case.shared, S, *ffn)

        if threads == 1:
            y, ysh, read = part((0, m, cfg.S))
        else:
            jobs = [(u, u + 1, 0) for u in range(m)] + [(0, 0, cfg.S)]
            with ThreadPoolExecutor(threads) as ex:
                parts = list(ex.map(part, jobs))
            y = np.zeros((n, cfg.K, cfg.d))
            for (u, _, _), (yp, _, _) in zip(jobs[:m], parts):
                for sl in un["perm"][un["offsets"][u]:un["offsets"][u + 1]]:
                    t, k = divmod(int(sl), cfg.K)
                    y[t, k] = yp[t, k]
            ysh = parts[-1][1]
            read = sum(p[2] for p in parts)
    else:
        evals = n * (cfg.K + cfg.S)
        if threads == 1:
            y, ysh, read = oracle.ffn_perslot(case.x, ids, case.expert, case.shared, cfg.S, *ffn)
        else:
            def part(job):  # slot (t, k), or the shared experts of token t (k = -1)
                t, k = job
                if k >= 0:
                    return oracle.ffn_perslot(case.x[t:t + 1], ids[t:t + 1, k:k + 1],
                                              case.expert, case.shared, 0, *ffn)
                return oracle.ffn_perslot(case.x[t:t + 1], ids[t:t + 1, :0], case.expert,
                                          case.shared, cfg.S, *ffn)

            jobs = [(t, k) for t in range(n) for k in range(cfg.K)] + \
                [(t, -1) for t in range(n) if cfg.S]
            with ThreadPoolExecutor(threads) as ex:
                parts = list(ex.map(part, jobs))
            y = np.zeros((n, cfg.K, cfg.d))
            ysh = np.zeros((n, cfg.S, cfg.d))
            for (t, k), (yp, yshp, _) in zip(jobs, parts):
                if k >= 0:
                    y[t, k] = yp[0, 0]
                else:
                    ysh[t] = yshp[0]
            read = sum(p[2] for p in parts)
    oracle.combine(y, gates, ysh if cfg.S else None)
    return time.perf_counter() - t0, read, evals


def _oracle_cases(cfg, ns, routing, cores):
    """The sampled passes (layer 0, window 0, seed 0) with every weight they
    read generated beforehand, outside the clock (numpy releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from synth import make_case

    cases = []
    for n in ns:
        case = make_case(cfg, n, routing, seed=0, window=0, layer=0)
        ids, _ = oracle.route_topk(case.logits, cfg.K)
        un = oracle.build_union(ids, cfg.E)
        gen = [int(e) for e in un["union_ids"]] + [cfg.E + s for s in range(cfg.S)]
        with ThreadPoolExecutor(cores) as ex:
            list(ex.map(case.expert, gen))
        cases.append((n, case, int(un["U"])))
    return cases


def _oracle_leg(cfg, cases, mode, threads, n_experts):
    tot_b, tot_t, per = 0, 0.0, {}
    for n, case, _ in cases:
        t, read, evals = _oracle_pass(cfg, case, mode, threads, n_experts)
        tot_b += read
        tot_t += t
        per["n=%d" % n] = {"experts": evals, "us_op": round(t * 1e6, 1),
                           "GBs": round(read / t / 1e9, 3)}
    return {"value": round(tot_b / tot_t / 1e9, 3), "s": round(tot_t, 2), "per_n": per}


def cpu_baseline(cfg, n_experts):
    """The oracle as it stands, timed on the host cores on one thread and on
    every core (BLAS one thread per call), with the core count:

    - the headline value: the deduplicating op on a bounded sample of the
      headline workload, the passes n = 1 and n = 8 (independent routing,
      layer 0), each capped at its first `n_experts` union experts (by
      default the whole union), GB/s on the union bytes read;
    - `perslot`: the per-slot op on the same passes, GB/s on requested bytes;
    - `olmoe`: the OLMoE-shaped bf16 layer at n = 1..8 (Markov p = 0.5), both
      ops, µs per op and GB/s.
    Weight generation is outside the clock; weight decode is inside."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from synth.configs import OLMOE

    cores = len(os.sched_getaffinity(0))
    head = _oracle_cases(cfg, (1, 8), "iid", cores)
    olm = _oracle_cases(OLMOE, range(1, 9), "markov:0.5", cores)
    res = {}
    with threadpool_limits(limits=1):
        for threads in (1, cores):
            res[("dedup", threads)] = _oracle_leg(cfg, head, "dedup", threads, n_experts)
            res[("perslot", threads)] = _oracle_leg(cfg, head, "perslot", threads, n_experts)
            res[("olmoe dedup", threads)] = _oracle_leg(OLMOE, olm, "dedup", threads, 64)
            res[("olmoe perslot", threads)] = _oracle_leg(OLMOE, olm, "perslot", threads, 64)
    for (leg, threads), r in res.items():
        log("cpu oracle, %s, %d thread(s): %s" % (leg, threads, json.dumps(r)))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    whole = all(min(U, n_experts) == U for _, _, U in head)
    scope = ("each pass whole (all %s union experts%s)"
             % ("/".join(str(U) for _, _, U in head),
                " + %d shared" % cfg.S if cfg.S else "") if whole else
             "each limited to its first %d union experts and every slot routed to them"
             % n_experts)
    sample = ("float64 numpy oracle (route, union, deduplicating FFN incl. fp8 weight decode, "
              "combine) on the %s layer, layer 0, independent routing, passes n=1 and n=8, %s; "
              "GB/s on the union bytes read; %d threads (one oracle call per union expert), "
              "BLAS one thread each" % (cfg.name, scope, cores))

    def both(leg):
        return {"value": res[(leg, cores)]["value"], "cores": cores,
                "per_n": res[(leg, cores)]["per_n"],
                "single_thread": {"value": res[(leg, 1)]["value"], "cores": 1,
                                  "per_n": res[(leg, 1)]["per_n"]}}

    out = {"value": res[("dedup", cores)]["value"], "unit": "GB/s", "cores": cores,
           "kind": "oracle", "cpu": model,
           "blas": ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()})),
           "sample": sample, "per_n": res[("dedup", cores)]["per_n"],
           "single_thread": {"value": res[("dedup", 1)]["value"], "cores": 1,
                             "per_n": res[("dedup", 1)]["per_n"]},
           "perslot": dict(both("perslot"), unit="GB/s on requested bytes",
                           sample="the same passes, per-slot op (one oracle call per slot)"),
           "olmoe": {"workload": "OLMoE-shaped bf16 layer, Markov p=0.5, layer 0, n=1..8",
                     "dedup": both("olmoe dedup"), "perslot": both("olmoe perslot")},
           "cpu_seconds": round(sum(r["s"] * (1 if th == 1 else cores)
                                    for (_, th), r in res.items()), 1)}
    return out


# ------------------------------------------------------------ other shapes
def shape_sweep(dev, reps=10):
    """The one-launch pass on the other layer shapes, deduplicating and per-slot:
    OLMoE with the other reuse probabilities of its recipe (p = 0, 0.8) and with
    independent routing; Qwen3-30B-A3B (router logits from AR(1) tokens);
    DeepSeek-V2-Lite (two shared experts, Markov p = 0.5, a 16-node draft tree);
    DeepSeek-V3 with 32-node draft trees.  Each point replays a graph of one pass
    per layer (layers alternate, so no pass finds its experts in the Infinity
    Cache); GB/s on union bytes (dedup) and on requested bytes (per-slot)."""
    import torch

    from synth.configs import DSV2LITE, DSV3, OLMOE, QWEN3
    plan = ((OLMOE, 4, (("markov:0.0", 8, False), ("markov:0.8", 8, False), ("iid", 8, False))),
            (QWEN3, 4, tuple(("logits_ar1", n, False) for n in (1, 2, 4, 8))),
            (DSV2LITE, 4, tuple(("markov:0.5", n, False) for n in (1, 2, 4, 8)) +
             (("markov:0.5", 16, True),)),
            (DSV3, 2, (("markov:0.5", 32, True), ("iid", 32, True))))
    out = {}
    for cfg, nl, points in plan:
        run = Runner(cfg, nl, dev)
        for routing, n, tree in points:
            ops = run.ops(routing, n, tree=tree)
            run.eager(ops)
            p = run.point(ops, reps)
            key = "%s %s n=%d%s" % (cfg.name, routing, n, " tree" if tree else "")
            out[key] = point_record(p)
            log("shape %s: %s" % (key, json.dumps(out[key])))
            del ops
        del run
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
    from moe_speculative_decoding_amd.layer import verify_layer, verify_layer_budget
    from synth.configs import DSV3, OLMOE

    plan = ((OLMOE, 8, "markov:0.5", 8, False, (8, 16, 24)),
            (DSV3, 2, "markov:0.5", 32, True, (32, 64)))
    out = {}
    for cfg, nl, routing, n, tree, budgets in plan:
        run = Runner(cfg, nl, dev)
        ops = run.ops(routing, n, tree=tree)

        def timed(call):
            for op in ops:
                call(op)
            torch.cuda.synchronize()
            for op in ops:
                if L.moe_get_error(op["buf"].ws) != L.MOE_OK:
                    raise RuntimeError("device error word set (%s n=%d)" % (cfg.name, n))
            outs = [op["buf"].out[:n].double().cpu() for op in ops]
            gates = [op["buf"].gates[:n].double().cpu() for op in ops]
            byt = sum(op["buf"].bytes.cpu().tolist()[0] for op in ops) / nl
            g = capture(lambda: [call(op) for op in ops])
            t = time_graph(g, nl, reps)
            del g
            return t, byt, outs, gates

        t0, b0, ref_out, ref_g = timed(
            lambda op: verify_layer(run.layers[op["layer"]], op["buf"], op["x"], op["logits"], n,
                                    L.MOE_MODE_DEDUP))
        base = "%s %s n=%d%s" % (cfg.name, routing, n, " tree" if tree else "")
        out[base + " no budget"] = {"union_MB": round(b0 / 1e6, 1), "us": round(1e6 * t0, 2),
                                    "GBs_union": round(b0 / t0 / 1e9, 1)}
        log("budget %s: %s" % (base, json.dumps(out[base + " no budget"])))
        for C in budgets:
            t, byt, outs, _ = timed(
                lambda op, C=C: verify_layer_budget(run.layers[op["layer"]], op["buf"], op["x"],
                                                    op["logits"], n, C, True))
            kept_mass = []
            for op in ops:  # the dropped share of gate mass, from the unbudgeted gates
                keep = (op["buf"].slot_rank[:n * cfg.K].cpu() >= 0).reshape(n, cfg.K).double()
                g = ref_g[op["layer"]]
                kept_mass.append(float((g * keep).sum() / g.sum()))
            dev_rel = [float(torch.linalg.norm(o - r) / torch.linalg.norm(r))
                       for o, r in zip(outs, ref_out)]
            key = "%s C=%d" % (base, C)
            out[key] = {"union_MB": round(byt / 1e6, 1), "us": round(1e6 * t, 2),
                        "GBs_union": round(byt / t / 1e9, 1),
                        "speedup_vs_no_budget": round(t0 / t, 3),
                        "gate_mass_dropped": round(1.0 - sum(kept_mass) / len(kept_mass), 4),
                        "out_rel_l2_vs_no_budget": round(sum(dev_rel) / len(dev_rel), 4)}
            log("budget %s: %s" % (key, json.dumps(out[key])))
        del ops, run
        torch.cuda.empty_cache()
    return out


def selection_sweep(dev, V_us):
    """Draft-tree selection ahead of the verify pass: EVICT truncation (cost
    table = the measured per-op times), EcoSpec selection and the offline
    Bellman draft-length policy; microseconds per call from graph replays."""
    import numpy as np
    import torch

    from moe_speculative_decoding_amd import _lib as L
    from synth.gen import draft_tree, expert_bitsets, predicted_sets, reference_sequence_inputs
    sel_ws = torch.zeros(256, dtype=torch.uint8, device=dev)
    out = {}
    for N in (32, 64, 1024):
        parent, q = draft_tree(N, 0)
        k = np.arange(1, N + 1)
        cost = np.interp(k + 1, np.arange(1, len(V_us) + 1), V_us)
        d_par, d_q = torch.from_numpy(parent).to(dev), torch.from_numpy(q).to(dev)
        d_c = torch.from_numpy(cost.astype(np.float32)).to(dev)
        order = torch.empty(N, dtype=torch.int32, device=dev)
        kb = torch.empty(1, dtype=torch.int32, device=dev)
        g = capture(lambda: [L.moe_evict_select(d_par, d_q, d_c, N, order, None, None, kb,
                                                    sel_ws, 256) for _ in range(8)])
        out["evict_N%d_us" % N] = round(1e6 * time_graph(g, 8, 20), 2)
        del g
    for N, nl, ne, kk, gamma in ((14, 16, 64, 8, 4), (64, 48, 128, 8, 16)):
        parent, q = draft_tree(N, 1)
        bits = expert_bitsets(predicted_sets(N, nl, ne, kk, 1, parent), nl, ne)
        d_par, d_q = torch.from_numpy(parent).to(dev), torch.from_numpy(q).to(dev)
        d_pred = torch.from_numpy(bits.view(np.int64)).to(dev)
        selv = torch.empty(gamma, dtype=torch.int32, device=dev)
        g = capture(lambda: [L.moe_ecospec_select(d_par, d_q, d_pred, None, N, bits.shape[1],
                                                      gamma, 0.1, selv, None, sel_ws, 256)
                                 for _ in range(8)])
        out["ecospec_N%d_L%d_E%d_g%d_us" % (N, nl, ne, gamma)] = round(1e6 * time_graph(g, 8, 20), 2)
        del g
    for N, Lmax in ((2048, 8), (2048, 12)):
        qv, cv = reference_sequence_inputs(N, Lmax, 0)
        d_q, d_c = torch.from_numpy(qv).to(dev), torch.from_numpy(cv).to(dev)
        dpv = torch.empty(N + 1, dtype=torch.float64, device=dev)
        kbv = torch.empty(N, dtype=torch.int32, device=dev)
        g = capture(lambda: [L.moe_bellman_policy(d_q, d_c, N, Lmax, dpv, kbv, sel_ws, 256)])
        t = time_graph(g, 1, 5)
        del g
        out["bellman_N%d_L%d_us" % (N, Lmax)] = round(1e6 * t, 1)
        out["bellman_N%d_L%d_mean_k" % (N, Lmax)] = round(float(kbv.double().mean()), 3)
    if L.moe_get_error(sel_ws) != L.MOE_OK:
        raise RuntimeError("selection kernels set the error word")
    log("selection: %s" % json.dumps(out))
    return out


def olmoe_detail(dev, nlayers, reps):
    """The OLMoE-shaped bf16 layer (E=64 K=8 d=2048 f=1024), Markov p = 0.5,
    n = 1, 2, 4, 8 over `nlayers` layers: both modes of the one-launch pass,
    the cost-model fit and the roofline of its deduplicating launches."""
    import torch

    from synth.configs import OLMOE
    run = Runner(OLMOE, nlayers, dev)
    ns = (1, 2, 4, 8)
    points, rec = {}, {}
    for n in ns:
        ops = run.ops("markov:0.5", n)
        run.eager(ops, chain_check=True)
        points[n] = run.point(ops, reps)
        rec["n=%d" % n] = point_record(points[n])
        log("olmoe n=%d %s" % (n, json.dumps(rec["n=%d" % n])))
        del ops
    b_e = run.layers[0].expert_bytes()
    tot_b = sum(points[n]["union_bytes"] for n in ns)
    tot_t = sum(points[n]["t_dedup"] for n in ns)
    out = {"workload": "OLMoE-shaped layer, bf16, E=64 K=8 d=2048 f=1024, Markov p=0.5, "
                       "%d layers" % nlayers,
           "points": rec, "fit": fits(points, ns, b_e, OLMOE.K, OLMOE.S),
           "GBs_dedup_union": round(tot_b / tot_t / 1e9, 1),
           "frac_dedup": round(tot_b / tot_t / 1e9 / PEAK_GBS, 4)}
    del run
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from moe_speculative_decoding_amd import _lib as L
    from moe_speculative_decoding_amd import costmodel as cm
    from moe_speculative_decoding_amd.layer import verify_layer_auto
    from synth.configs import DSV3, OLMOE

    dev = "cuda:0"
    torch.cuda.set_device(0)
    DEDUP, SLOT = L.MOE_MODE_DEDUP, L.MOE_MODE_PERSLOT

    tree = False
    if args.workload == "dsv3tree" and not (args.counters or args.profile_step):
        print("--workload dsv3tree is for --counters and --profile-step", file=sys.stderr)
        sys.exit(2)
    if args.workload == "olmoe":
        cfg, nlayers, routings, ns = OLMOE, args.olmoe_layers, ("markov:0.5",), (1, 2, 4, 8)
    elif args.workload == "dsv3tree":
        cfg, nlayers, routings, ns, tree = DSV3, 2, ("markov:0.5", "iid"), (32,), True
    else:
        cfg, nlayers, routings, ns = DSV3, args.layers, HEADLINE_ROUTINGS, HEADLINE_NS
    log("generating %d layers of %s weights on the device" % (nlayers, cfg.name))
    run = Runner(cfg, nlayers, dev)
    keys = [(routing, n) for routing in routings for n in ns]
    by_key = {k: run.ops(*k, tree=tree) for k in keys}
    ops = [op for k in keys for op in by_key[k]]
    light = args.profile_step or args.counters
    # (profile-step mode: deduplicating launches only, so the kernel trace
    # holds nothing but the step's launches and their eager references)
    run.eager(ops, chain_check=not light, both=not args.profile_step)
    step_union_bytes = sum(op["union_bytes"] for op in ops)

    if args.counters:
        # under rocprofv3 --pmc: calibration copies, then one dispatch per
        # operation and mode, in this order
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        seq = []
        for mode, name in ((DEDUP, "dedup"), (SLOT, "perslot")):
            for op in ops:
                run.call(op, mode)
                torch.cuda.synchronize()
                seq.append({"mode": name, "routing": op["routing"], "n": op["n"],
                            "layer": op["layer"], "U": op["U"], "union_bytes": op["union_bytes"],
                            "requested_bytes": op["requested_bytes"]})
        manifest = {"workload": args.workload, "copy_bytes": src.numel() * 4, "copies": 3,
                    "kernel": "layer_kernel", "expert_bytes": run.layers[0].expert_bytes(),
                    "K": cfg.K, "S": cfg.S, "launches": seq}
        with open(args.counters, "w") as fh:
            json.dump(manifest, fh)
        log("counter mode: %d launches written to %s" % (len(seq), args.counters))
        return

    # ---------------------------------------------------------- the step
    log("capturing one step (%d operations, one launch each) in a graph" % len(ops))
    g_step = capture(lambda: [run.call(op, DEDUP) for op in ops])
    for rep in range(3):  # replays must reproduce the eager results exactly
        for op in ops:
            op["buf"].out.zero_()
        torch.cuda.synchronize()
        g_step.replay()
        torch.cuda.synchronize()
        for op in ops:
            if L.moe_get_error(op["buf"].ws) != L.MOE_OK:
                raise RuntimeError("device error word set in replay %d" % rep)
            if not torch.equal(op["buf"].out[:op["n"]], op["out_eager"]):
                raise RuntimeError("graph replay %d differs from the eager pass" % rep)
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        g_step.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # the step's launches back to back on the launch stream, HIP events around them
    launch_s = e0.elapsed_time(e1) * 1e-3 / (args.steps * len(ops))
    value = step_union_bytes / (ms_per_step * 1e-3) / 1e9
    log("step: %.3f ms, %.1f GB/s on union bytes" % (ms_per_step, value))
    if args.profile_step:
        log("profile-step mode: %d replays of %d launches, nothing else timed"
            % (args.steps + args.warmup + 3, len(ops)))
        if args.step_manifest:
            with open(args.step_manifest, "w") as fh:
                json.dump({"workload": args.workload, "ms_per_step": ms_per_step,
                           "ops": [{"routing": op["routing"], "n": op["n"], "layer": op["layer"],
                                    "U": op["U"], "union_bytes": op["union_bytes"]}
                                   for op in ops]}, fh)
        return
    del g_step

    # ------------------------------------------- per (routing, n), both modes
    points = {k: run.point(by_key[k], args.reps) for k in keys}
    detail = {}
    for routing in routings:
        for n in ns:
            detail["%s n=%d" % (routing, n)] = point_record(points[(routing, n)])
            log("%s n=%d %s" % (routing, n, json.dumps(detail["%s n=%d" % (routing, n)])))
    b_e = run.layers[0].expert_bytes()
    fit = {routing: fits({n: points[(routing, n)] for n in ns}, ns, b_e, cfg.K, cfg.S)
           for routing in routings}

    # ---- mode dispatch (expert-bytes page, Eq. (7)): every pass takes the mode
    # its n's measured r picks, decided on the device from its own union
    r_of = {k: cm.aggregate([points[k]])["r"] for k in keys}
    mode_out = torch.zeros(len(ops), dtype=torch.int32, device=dev)

    def auto_call(i, op):
        verify_layer_auto(run.layers[op["layer"]], op["buf"], op["x"], op["logits"], op["n"],
                          r_of[(op["routing"], op["n"])], mode_out[i:i + 1])

    g_auto = capture(lambda: [auto_call(i, op) for i, op in enumerate(ops)])
    ms_auto = time_graph(g_auto, 1, max(2, args.reps // 4)) * 1e3
    del g_auto
    picked = mode_out.cpu().tolist()
    dispatch = {"rule": "dedup iff u(n) < r(n) (Eq. (7)), decided on the device from each "
                        "pass's union with the measured r of its (routing, n)",
                "ms_per_step_auto": round(ms_auto, 4), "ms_per_step_dedup": round(ms_per_step, 4),
                "dedup_passes": sum(1 for m in picked if m == DEDUP), "passes": len(picked)}
    # best draft length from V(k) = tau(k + 1) of the Markov routing
    model = {}
    for n in ns:
        p = points[(routings[-1], n)]
        a = cm.aggregate([p])
        model[n] = p["t_dedup"] if cm.dedup_faster(a["u"], a["r"]) else p["t_slot"]
    V = [model[k + 1] for k in range(len(ns))]
    draft = {"V_us": [round(1e6 * v, 2) for v in V], "a0": round(cm.a0(V), 4),
             "step_points": [[round(a, 4), k] for a, k in cm.step_points(V)],
             "k_star": {"a=%.1f" % a: cm.best_draft_length(V, a) for a in (0.3, 0.5, 0.7, 0.8, 0.9)},
             "reading": "V(k) = time of one MoE layer op at n = k+1 (%s routing) in the mode "
                        "Eq. (7) picks; geometric acceptance, T_a(k) = sum_{j<=k} a^j / V(k)"
                        % routings[-1]}
    log("dispatch: %s" % json.dumps(dispatch))
    log("draft length: %s" % json.dumps(draft))

    # ---- roofline of the dominant kernel: the deduplicating layer_kernel launches
    # of the step, algorithmic bytes (union expert bytes) per launch over the
    # average launch duration inside the step replays
    achieved = step_union_bytes / len(ops) / launch_s / 1e9
    traffic, trec = measured_traffic(args.workload)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
                "kernel": "layer_kernel (moe_verify_layer, deduplicating): the %d launches of "
                          "the step, HIP events on the launch stream around %d step replays"
                          % (len(ops), args.steps),
                "bytes_per_launch": "(U + S) * b, b = 3*d*f*1 B + 3*(d/128)*(f/128)*4 B of "
                                    "scales = %d B; mean %.0f B" % (b_e, step_union_bytes / len(ops)),
                "launch_us_mean": round(1e6 * launch_s, 2),
                "launch_us": {"%s n=%d" % k: round(1e6 * points[k]["t_dedup"], 2) for k in keys}}
    if trec is not None:
        roofline["counters"] = {"dedup_fetch_over_union": trec["dedup"].get("fetch_over_union"),
                                "perslot_fetch_over_requested":
                                    trec.get("perslot", {}).get("fetch_over_requested"),
                                "current": traffic is not None}
    del by_key, ops
    del run
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_shapes:
        extra["olmoe"] = olmoe_detail(dev, args.olmoe_layers, args.reps)
        extra["shapes"] = shape_sweep(dev)
        extra["budget"] = budget_sweep(dev)
        extra["selection"] = selection_sweep(dev, draft["V_us"])

    cpu = None if args.no_cpu else cpu_baseline(cfg, args.cpu_experts)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 weights x bf16 tokens, fp32 accumulate" if cfg.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": "%s-shaped MoE layer verify op (route, union, deduplicating SwiGLU "
                               "experts, combine; one launch per op), E=%d K=%d d=%d f=%d, %s; "
                               "n=%s; routing %s; %d layers; HIP-graph step"
                               % (cfg.name, cfg.E, cfg.K, cfg.d, cfg.f,
                                  "fp8 E4M3FN weights with 128x128 fp32 block scales, bf16 tokens"
                                  if cfg.fp8 else "bf16 weights and tokens",
                                  ",".join(str(n) for n in ns), " and ".join(routings), nlayers),
                   "global_batch": sum(ns) * len(routings) * nlayers, "seq_len": 1,
                   "parallelism": "none"},
        "roofline": roofline, "cpu_baseline": cpu, "detail": detail, "fit": fit,
        "dispatch": dispatch, "draft_length": draft,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
