"""Shared helpers of the GPU parity tests: upload a synth case, run the HIP path
through the C ABI, and compare with the oracle.

Tolerances
- ids, union, permutation, byte counts: bit-exact.
- gates: fp32 softmax against float64: |err| <= 1e-6 + 1e-5 |ref|.
- the one-launch pass (moe_verify_layer) against the chain of entry points:
  bit-exact in every output (same arithmetic in the same order), on two
  calls in a row on one workspace (the first leaves its counters zero).
- expert outputs, relative L2 per slot (and over the whole output):
  the contractual bound of the layer (1e-5 f32, 1e-2 bf16, 3e-2 fp8) and a
  derived bound: the HIP path rounds the intermediate h = silu(a) * v to
  bf16 once (relative error uniform in +-2^-9, RMS 2^-9 / sqrt(3) = 1.1e-3)
  and accumulates in fp32, so bf16/fp8 weights stay below 4e-3; f32 weights
  keep h in fp32 (1e-5).  Elementwise, |err| <= 8 * bound * RMS(ref slot).
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np
import torch

import oracle
from moe_speculative_decoding_amd import _lib as L
from moe_speculative_decoding_amd.layer import (DeviceLayer, VerifyBuffers, to_device, verify_layer,
                                                verify_pass)

DEV = "cuda:0"


def derived_bound(cfg) -> float:
    return 1e-5 if cfg.w_dtype == "f32" else 4e-3


def upload_layer(case, experts: Optional[Iterable[int]] = None) -> DeviceLayer:
    """Device copy of the case's layer; experts not listed stay zero."""
    cfg = case.cfg
    want = range(cfg.E) if experts is None else sorted(set(int(e) for e in experts))
    sample = case.expert(next(iter(want)) if len(want) else 0)
    routed = {k: np.zeros((cfg.E,) + v.shape, dtype=v.dtype) for k, v in sample.items()}
    for e in want:
        for k, v in case.expert(e).items():
            routed[k][e] = v
    shared = None
    if cfg.S:
        shared = {k: np.stack([case.shared(s)[k] for s in range(cfg.S)]) for k in sample}
    return DeviceLayer.from_arrays(cfg, routed, shared, DEV)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (den if den > 0 else 1.0)


def check_vectors(got: np.ndarray, ref: np.ndarray, tol: float, what: str) -> float:
    """Per-row (last axis) relative L2 and elementwise check; returns the worst row error."""
    got = got.reshape(-1, got.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    worst = 0.0
    for i in range(ref.shape[0]):
        e = rel_l2(got[i], ref[i])
        worst = max(worst, e)
        rms = math.sqrt(float(np.mean(ref[i] ** 2)))
        assert e <= tol, "%s row %d: rel L2 %.3e > %.1e" % (what, i, e, tol)
        assert np.max(np.abs(got[i] - ref[i])) <= 8 * tol * rms + 1e-30, \
            "%s row %d: elementwise error too large" % (what, i)
    return worst


def run_case(case, modes=("dedup", "perslot"), ref=None, experts=None,
             fused: bool = True) -> Dict[str, object]:
    """Run the whole pass on the GPU in each mode and compare with the oracle."""
    cfg = case.cfg
    n = case.n
    if ref is None:
        ref = oracle.verify_op(case, "dedup")
    U = int(ref["union"]["U"])
    layer = upload_layer(case, ref["union"]["union_ids"][:U] if experts is None else experts)
    x = to_device(case.x, DEV)
    logits = to_device(case.logits, DEV)
    tol = cfg.tolerance
    tight = min(tol, derived_bound(cfg))
    report = {"U": U}
    for mode in modes:
        m = L.MOE_MODE_DEDUP if mode == "dedup" else L.MOE_MODE_PERSLOT
        buf = VerifyBuffers(layer, n, DEV)
        print("case %s n=%d routing=%s seed=%d mode=%s" % (cfg.name, n, case.routing, case.seed, mode),
              flush=True)
        verify_pass(layer, buf, x, logits, n, m)
        torch.cuda.synchronize()
        assert L.moe_get_error(buf.ws) == L.MOE_OK
        ids = buf.ids[:n].cpu().numpy()
        assert np.array_equal(ids, ref["ids"]), "ids differ"
        gates = buf.gates[:n].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(gates - ref["gates"]) <= 1e-6 + 1e-5 * np.abs(ref["gates"])), "gates"
        if mode == "dedup":
            un = ref["union"]
            assert int(buf.U.item()) == U
            assert np.array_equal(buf.union_ids.cpu().numpy()[:len(un["union_ids"])], un["union_ids"])
            assert np.array_equal(buf.offsets.cpu().numpy()[:len(un["offsets"])], un["offsets"])
            assert np.array_equal(buf.perm[:n * cfg.K].cpu().numpy(), un["perm"])
            assert np.array_equal(buf.slot_rank[:n * cfg.K].cpu().numpy(), un["slot_rank"])
        b = buf.bytes.cpu().numpy().astype(np.uint64)
        expect0 = ref["union_bytes"] if mode == "dedup" else ref["requested_bytes"]
        assert int(b[0]) == expect0 and int(b[1]) == ref["requested_bytes"], "byte counts"
        y = buf.y_slots[:n].cpu().numpy()
        w = check_vectors(y, ref["y_slots"], tight, mode + " y_slots")
        if cfg.S:
            check_vectors(buf.y_shared[:n, :cfg.S].cpu().numpy(), ref["y_shared"], tight,
                          mode + " y_shared")
        out = buf.out[:n].float().cpu().numpy()
        check_vectors(out, ref["out"], tight, mode + " out")
        report[mode] = w
        if fused:
            check_fused_matches(layer, buf, x, logits, n, m, mode)
    return report


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint8)


def check_fused_matches(layer: DeviceLayer, chain: VerifyBuffers, x, logits, n: int, m: int,
                        mode: str) -> None:
    """moe_verify_layer reproduces the chain's outputs bit for bit, twice."""
    K, S = layer.K, layer.S
    buf = VerifyBuffers(layer, n, DEV, out_dtype=chain.out_dtype)
    for call in range(2):
        print("  fused call %d mode=%s" % (call, mode), flush=True)
        buf.out.zero_()
        buf.y_slots.zero_()
        verify_layer(layer, buf, x, logits, n, m)
        torch.cuda.synchronize()
        assert L.moe_get_error(buf.ws) == L.MOE_OK, "fused: device error"
        pairs = [("ids", buf.ids[:n], chain.ids[:n]), ("gates", buf.gates[:n], chain.gates[:n]),
                 ("bytes", buf.bytes, chain.bytes), ("y_slots", buf.y_slots[:n], chain.y_slots[:n]),
                 ("out", buf.out[:n], chain.out[:n])]
        if S:
            pairs.append(("y_shared", buf.y_shared[:n, :S], chain.y_shared[:n, :S]))
        if mode == "dedup":
            pairs += [("U", buf.U, chain.U), ("union_ids", buf.union_ids, chain.union_ids),
                      ("offsets", buf.offsets, chain.offsets),
                      ("perm", buf.perm[:n * K], chain.perm[:n * K]),
                      ("slot_rank", buf.slot_rank[:n * K], chain.slot_rank[:n * K])]
        for name, a, b in pairs:
            assert np.array_equal(_bits(a), _bits(b)), "fused %s call %d: %s differs" % (mode, call, name)
    # outputs kept in the workspace: the same layer output
    buf.out.zero_()
    verify_layer(layer, buf, x, logits, n, m, keep=False)
    torch.cuda.synchronize()
    assert L.moe_get_error(buf.ws) == L.MOE_OK
    assert np.array_equal(_bits(buf.out[:n]), _bits(chain.out[:n])), "fused (workspace outputs)"
