"""GPU: many replays of full-size one-launch passes, each bit for bit equal to
the eager pass.

The one-launch pass hands work between workgroups through flags tagged with
the call's epoch; a race in that hand-over (a DOWN range reading H before its
owners wrote it, a combine reading a slot row before its DOWN range stored
it) would show as a replay whose outputs differ from the eager ones now and
then.  This test captures sixteen passes of the benchmark's own layers in
one HIP graph: the DeepSeek-V3-shaped fp8 layer at n = 1, 2, 3, 6, 8 and
draft trees of 16 and 32 nodes, per-slot at n = 8, and the OLMoE-shaped bf16
layer at n = 1, 2, 4, 8 (two reuse levels) and per-slot at n = 8; and two
more forms of the pass at full size, the expert budget (32-node tree, C = 32)
and the mode chosen on the device (n = 4).  It replays the graph a thousand
times, clears the outputs before each replay (outside the graph), and checks
the error word, the layer output, the slot outputs and the chosen mode of
every pass after every replay.
"""
import pytest
import torch

from synth import make_case
from synth.configs import DSV3, OLMOE

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from moe_speculative_decoding_amd import _lib as L  # noqa: E402
from moe_speculative_decoding_amd.layer import (  # noqa: E402
    DeviceLayer, VerifyBuffers, to_device, verify_layer, verify_layer_auto, verify_layer_budget)
from synth.gen import device_layer_weights  # noqa: E402
from gpu_harness import DEV  # noqa: E402

REPLAYS = 1000
DEDUP, PERSLOT = L.MOE_MODE_DEDUP, L.MOE_MODE_PERSLOT
BUDGET, AUTO = "budget", "auto"
PASSES = [  # (config, n, routing, tree, mode)
    (DSV3, 1, "iid", False, DEDUP), (DSV3, 2, "iid", False, DEDUP),
    (DSV3, 3, "markov:0.5", False, DEDUP), (DSV3, 6, "markov:0.5", False, DEDUP),
    (DSV3, 8, "iid", False, DEDUP), (DSV3, 16, "iid", True, DEDUP),
    (DSV3, 32, "markov:0.5", True, DEDUP), (DSV3, 8, "iid", False, PERSLOT),
    (OLMOE, 1, "markov:0.5", False, DEDUP), (OLMOE, 2, "markov:0.5", False, DEDUP),
    (OLMOE, 4, "markov:0.5", False, DEDUP), (OLMOE, 8, "markov:0.5", False, DEDUP),
    (OLMOE, 8, "markov:0.0", False, DEDUP), (OLMOE, 8, "markov:0.5", False, PERSLOT),
    (DSV3, 32, "markov:0.5", True, BUDGET), (DSV3, 4, "iid", False, AUTO),
]


def _call(layer, buf, x, lg, n, mode):
    if mode == BUDGET:
        verify_layer_budget(layer, buf, x, lg, n, 32, True)
    elif mode == AUTO:
        verify_layer_auto(layer, buf, x, lg, n, 0.95, buf.mode_out)
    else:
        verify_layer(layer, buf, x, lg, n, mode)


def test_full_size_graph_replays_match_eager():
    layers = {}
    for cfg in (DSV3, OLMOE):
        w = device_layer_weights(cfg, seed=0, layer=0, device=DEV)
        layers[cfg.name] = DeviceLayer(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype,
                                       cfg.x_dtype, w, None)
    plan = []
    for cfg, n, routing, tree, mode in PASSES:
        case = make_case(cfg, n, routing, seed=7, window=0, layer=0, tree=tree)
        kind = {DEDUP: "dedup", PERSLOT: "perslot"}.get(mode, mode)
        name = "%s %s n=%d %s" % (cfg.name, routing, n, kind)
        buf = VerifyBuffers(layers[cfg.name], n, DEV)
        buf.mode_out = torch.zeros(1, dtype=torch.int32, device=DEV)
        plan.append((name, n, mode, layers[cfg.name], to_device(case.x, DEV),
                     to_device(case.logits, DEV), buf))

    refs = []
    for name, n, mode, layer, x, lg, buf in plan:
        buf.out.zero_()
        buf.y_slots.zero_()
        _call(layer, buf, x, lg, n, mode)
        torch.cuda.synchronize()
        assert L.moe_get_error(buf.ws) == L.MOE_OK, name
        refs.append((buf.out.clone(), buf.y_slots.clone(), buf.mode_out.clone()))

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for name, n, mode, layer, x, lg, buf in plan:
                _call(layer, buf, x, lg, n, mode)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(REPLAYS):
        for *_, buf in plan:
            buf.out.zero_()  # fill kernels outside the graph
            buf.y_slots.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for (name, n, mode, layer, x, lg, buf), (ro, ry, rm) in zip(plan, refs):
            assert L.moe_get_error(buf.ws) == L.MOE_OK, (rep, name)
            assert torch.equal(buf.out, ro), (rep, name, "out")
            assert torch.equal(buf.y_slots, ry), (rep, name, "y_slots")
            assert torch.equal(buf.mode_out, rm), (rep, name, "mode")
        if rep % 250 == 0:
            print("replay %d of %d" % (rep, REPLAYS), flush=True)
    del graph
