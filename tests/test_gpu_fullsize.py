"""GPU parity at the benchmark's full layer sizes, in the launches the
benchmark times (the one-launch pass, moe_verify_layer, deduplicating and
per-slot, and its budgeted form), on sampled outputs.

The layers are the benchmark's own: every expert of the layer drawn on the
device (synth.gen.device_layer_weights), so the DeepSeek-V3-shaped layer holds
all 256 fp8 experts (11 GB).  The oracle checks routing, the union arrays and
the byte counters in full (bit for bit), and the slot outputs and layer output
of a few sampled tokens (every token of the OLMoE-shaped passes, which the
benchmark times at n = 1, 2, 4 and 8): for each sampled token its K experts (and the shared experts) are copied back
from the device and evaluated by the oracle in float64.  Tolerances as in
``gpu_harness`` (contractual bound and the derived bf16-rounding bound).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import make_case
from synth.configs import DSV2LITE, DSV3, OLMOE, QWEN3
from synth.gen import device_layer_weights

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from moe_speculative_decoding_amd import _lib as L  # noqa: E402
from moe_speculative_decoding_amd.layer import (  # noqa: E402
    DeviceLayer, VerifyBuffers, to_device, verify_layer)
from gpu_harness import DEV, check_vectors, derived_bound  # noqa: E402

_NAMES = ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")


def _expert_to_host(w, e, cfg):
    stored = {}
    for k in _NAMES:
        if k in w:
            a = w[k][e].cpu().numpy()
            stored[k] = a.view(np.uint16) if (cfg.w_dtype == "bf16" and a.dtype == np.int16) else a
    return oracle.DecodedExpert(stored, cfg.w_dtype)


@pytest.mark.parametrize("cfg,n,routing,tree,tokens,mode", [
    (OLMOE, 8, "markov:0.5", False, range(8), "dedup"),
    (OLMOE, 4, "markov:0.5", False, range(4), "dedup"),
    (OLMOE, 2, "markov:0.5", False, range(2), "dedup"),
    (OLMOE, 1, "markov:0.5", False, (0,), "dedup"),
    (OLMOE, 8, "markov:0.5", False, (0, 7), "perslot"),
    (OLMOE, 1, "markov:0.5", False, (0,), "perslot"),
    (QWEN3, 8, "logits_ar1", False, (0, 5), "dedup"),
    (QWEN3, 1, "logits_ar1", False, (0,), "dedup"),
    (DSV2LITE, 1, "markov:0.5", False, (0,), "dedup"),
    (DSV2LITE, 8, "markov:0.5", False, (2, 6), "dedup"),
    (DSV2LITE, 16, "markov:0.5", True, (0, 9, 15), "dedup"),
    (DSV3, 1, "iid", False, (0,), "dedup"),
    (DSV3, 2, "iid", False, (0, 1), "dedup"),         # the two-token tile
    (DSV3, 3, "markov:0.5", False, (0, 2), "dedup"),  # the four-token tile, one row short
    (DSV3, 4, "iid", False, (1, 3), "dedup"),
    (DSV3, 6, "iid", False, (5,), "dedup"),
    (DSV3, 8, "iid", False, (0, 7), "dedup"),
    (DSV3, 8, "markov:0.5", False, (4,), "dedup"),
    (DSV3, 32, "markov:0.5", True, (0, 17, 31), "dedup"),
    (QWEN3, 8, "logits_ar1", False, (3,), "perslot"),
    (DSV2LITE, 16, "markov:0.5", True, (4, 12), "perslot"),
    (DSV3, 2, "markov:0.5", False, (1,), "perslot"),
    (DSV3, 8, "iid", False, (2,), "perslot"),
    (DSV3, 32, "markov:0.5", True, (5, 26), "perslot"),
])
def test_one_launch_pass_full_size_sampled(cfg, n, routing, tree, tokens, mode):
    print("full size %s n=%d routing=%s tree=%s %s" % (cfg.name, n, routing, tree, mode),
          flush=True)
    dedup = mode == "dedup"
    w = device_layer_weights(cfg, seed=0, layer=0, device=DEV)
    sh = device_layer_weights(cfg, seed=0, layer=0, device=DEV, shared=True) if cfg.S else None
    layer = DeviceLayer(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype, cfg.x_dtype, w, sh)
    case = make_case(cfg, n, routing, seed=0, window=0, layer=0, tree=tree)
    buf = VerifyBuffers(layer, n, DEV)
    verify_layer(layer, buf, to_device(case.x, DEV), to_device(case.logits, DEV), n,
                 L.MOE_MODE_DEDUP if dedup else L.MOE_MODE_PERSLOT)
    torch.cuda.synchronize()
    assert L.moe_get_error(buf.ws) == L.MOE_OK

    ids, gates = oracle.route_topk(case.logits, cfg.K)
    assert np.array_equal(buf.ids[:n].cpu().numpy(), ids)
    g_dev = buf.gates[:n].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(g_dev - gates) <= 1e-6 + 1e-5 * np.abs(gates))
    un = oracle.build_union(ids, cfg.E)
    U = un["U"]
    if dedup:  # the per-slot pass leaves the union arrays alone
        assert int(buf.U.item()) == U
        assert np.array_equal(buf.union_ids.cpu().numpy()[:len(un["union_ids"])],
                              un["union_ids"])
        assert np.array_equal(buf.offsets.cpu().numpy()[:len(un["offsets"])], un["offsets"])
        assert np.array_equal(buf.perm[:n * cfg.K].cpu().numpy(), un["perm"])
        assert np.array_equal(buf.slot_rank[:n * cfg.K].cpu().numpy(), un["slot_rank"])
    ub, rb = oracle.byte_counts(cfg.d, cfg.f, cfg.w_dtype, cfg.K, cfg.S, n, U)
    b = buf.bytes.cpu().numpy()
    assert int(b[0]) == (ub if dedup else rb) and int(b[1]) == rb

    tight = min(cfg.tolerance, derived_bound(cfg))
    xs = oracle.decode_x(case.x, cfg.x_dtype)
    y_dev = buf.y_slots[:n].cpu().numpy()
    ysh_dev = buf.y_shared[:n, :cfg.S].cpu().numpy() if cfg.S else None
    out_dev = buf.out[:n].float().cpu().numpy()
    decoded = {}
    shared = [_expert_to_host(sh, s_, cfg) for s_ in range(cfg.S)] if cfg.S else []
    for t in tokens:
        y_ref = np.zeros((cfg.K, cfg.d))
        for k in range(cfg.K):
            e = int(ids[t, k])
            if e not in decoded:
                decoded[e] = _expert_to_host(w, e, cfg)
            y_ref[k] = oracle.swiglu(xs[t], decoded[e])
        check_vectors(y_dev[t], y_ref, tight, "%s token %d y_slots" % (cfg.name, t))
        out_ref = (gates[t][:, None] * y_ref).sum(axis=0)
        for s_, ex in enumerate(shared):
            ysh = oracle.swiglu(xs[t], ex)
            check_vectors(ysh_dev[t, s_][None, :], ysh[None, :], tight,
                          "%s token %d y_shared %d" % (cfg.name, t, s_))
            out_ref = out_ref + ysh
        check_vectors(out_dev[t][None, :], out_ref[None, :], tight, "%s token %d out" % (cfg.name, t))
    del w, sh, layer, buf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg,n,routing,tree,C,tokens", [
    (OLMOE, 8, "markov:0.5", False, 16, range(8)),
    (OLMOE, 8, "markov:0.5", False, 24, (0, 4, 7)),
    (OLMOE, 8, "markov:0.5", False, 8, (1, 6)),
    (DSV3, 32, "markov:0.5", True, 32, (0, 17, 31)),
    (DSV3, 32, "markov:0.5", True, 64, (3, 30)),
])
def test_one_launch_budget_full_size_sampled(cfg, n, routing, tree, C, tokens):
    """The budgeted one-launch pass (moe_verify_layer_budget, kept gates
    renormalised) on the benchmark's budget sweep layers: routing, the kept
    union, gates and byte counters against the oracle's budget
    (oracle.apply_budget) in full, slot and layer outputs of sampled tokens
    against the oracle on the experts copied back, dropped slots zero."""
    from moe_speculative_decoding_amd.layer import verify_layer_budget
    print("full size budget %s n=%d C=%d" % (cfg.name, n, C), flush=True)
    case = make_case(cfg, n, routing, seed=0, window=0, layer=0, tree=tree)
    ids, gates = oracle.route_topk(case.logits, cfg.K)
    un = oracle.build_union(ids, cfg.E)
    bud = oracle.apply_budget(ids, gates, un, C, True)
    sc = np.sort(bud["scores"].astype(np.float64))[::-1]
    # no contribution within float32 reach of the cut: the device sums its own
    # float32 gates in float32, the oracle its float64 gates in float64
    assert C >= len(sc) or sc[C - 1] - sc[C] > 1e-5 * n, "near-tie at the cut: another seed"
    w = device_layer_weights(cfg, seed=0, layer=0, device=DEV)
    sh = device_layer_weights(cfg, seed=0, layer=0, device=DEV, shared=True) if cfg.S else None
    layer = DeviceLayer(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype, cfg.x_dtype, w, sh)
    buf = VerifyBuffers(layer, n, DEV)
    buf.y_slots.fill_(5.0)  # dropped rows must come back zero
    verify_layer_budget(layer, buf, to_device(case.x, DEV), to_device(case.logits, DEV), n, C,
                        True)
    torch.cuda.synchronize()
    assert L.moe_get_error(buf.ws) == L.MOE_OK

    assert np.array_equal(buf.ids[:n].cpu().numpy(), ids)
    U = bud["U"]
    assert U == min(C, un["U"])
    assert int(buf.U.item()) == U
    for key in ("union_ids", "offsets"):
        got = getattr(buf, key).cpu().numpy()[:len(bud[key])]
        assert np.array_equal(got, bud[key]), key
    assert np.array_equal(buf.perm[:n * cfg.K].cpu().numpy(), bud["perm"])
    assert np.array_equal(buf.slot_rank[:n * cfg.K].cpu().numpy(), bud["slot_rank"])
    g_dev = buf.gates[:n].cpu().numpy().astype(np.float64)
    g_ref = bud["gates"]
    assert np.all(np.abs(g_dev - g_ref) <= 1e-6 + 1e-5 * np.abs(g_ref)), "gates"
    assert np.array_equal(g_dev == 0.0, g_ref == 0.0)
    ub, rb = oracle.byte_counts(cfg.d, cfg.f, cfg.w_dtype, cfg.K, cfg.S, n, U)
    b = buf.bytes.cpu().numpy()
    assert int(b[0]) == ub and int(b[1]) == rb

    tight = min(cfg.tolerance, derived_bound(cfg))
    keep = bud["slot_rank"].reshape(n, cfg.K) >= 0
    xs = oracle.decode_x(case.x, cfg.x_dtype)
    y_dev = buf.y_slots[:n].cpu().numpy()
    assert np.all(y_dev[~keep] == 0.0), "dropped slots must have zero rows"
    out_dev = buf.out[:n].float().cpu().numpy()
    decoded = {}
    shared = [_expert_to_host(sh, s_, cfg) for s_ in range(cfg.S)] if cfg.S else []
    for t in tokens:
        y_ref = np.zeros((cfg.K, cfg.d))
        for k in range(cfg.K):
            if not keep[t, k]:
                continue
            e = int(ids[t, k])
            if e not in decoded:
                decoded[e] = _expert_to_host(w, e, cfg)
            y_ref[k] = oracle.swiglu(xs[t], decoded[e])
        if keep[t].any():
            check_vectors(y_dev[t][keep[t]], y_ref[keep[t]], tight,
                          "%s token %d kept y_slots" % (cfg.name, t))
        out_ref = (g_ref[t][:, None] * y_ref).sum(axis=0)
        for s_, ex in enumerate(shared):
            out_ref = out_ref + oracle.swiglu(xs[t], ex)
        check_vectors(out_dev[t][None, :], out_ref[None, :], tight,
                      "%s token %d budget out" % (cfg.name, t))
    del w, sh, layer, buf
    torch.cuda.empty_cache()
