"""GPU: the one-launch pass captured in a HIP graph and replayed.

The benchmark times graph replays, so a replay must give what an eager call
gives.  The pass keeps no host-side state between calls: each call takes its
tag from the workspace's epoch word and retires it at its end, so the
hand-over flags of one replay never satisfy the waits of the next.  This test
captures passes of several sizes (deduplicating, per-slot, budgeted, mode
chosen on the device) into one graph, replays it several times with eager
work and synchronisations in between, clears every output before each
replay (outside the graph), and checks every replay bit for bit against the
eager calls.
"""
import numpy as np
import pytest
import torch

from synth import make_case
from synth.configs import LayerConfig

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from moe_speculative_decoding_amd import _lib as L  # noqa: E402
from moe_speculative_decoding_amd.layer import (  # noqa: E402
    VerifyBuffers, to_device, verify_layer, verify_layer_auto, verify_layer_budget)
from gpu_harness import DEV, _bits, upload_layer  # noqa: E402

GRAPH_BF16 = LayerConfig(name="graph_bf16", cfg_id=84, E=24, K=4, d=264, f=136, S=1,
                         w_dtype="bf16", x_dtype="bf16", n_values=(1, 5, 8),
                         routing=("markov:0.5",), tolerance=1e-2)

_OUTS = ("out", "y_slots", "ids", "gates", "U", "union_ids", "offsets", "perm", "slot_rank",
         "bytes")


def _clear(buf):
    for name in _OUTS:
        getattr(buf, name).zero_()  # a fill kernel, not a memset node
    buf.y_shared.zero_()


def _snapshot(buf, n):
    snap = {name: _bits(getattr(buf, name)) for name in _OUTS}
    snap["y_shared"] = _bits(buf.y_shared[:n])
    return snap


def test_one_launch_pass_graph_replays_match_eager():
    case0 = make_case(GRAPH_BF16, 8, None, seed=41)
    layer = upload_layer(case0)  # every expert of the layer
    r_auto = 0.7
    plan = []  # (name, n, call)
    for n in (1, 5, 8):
        case = make_case(GRAPH_BF16, n, None, seed=50 + n)
        x, lg = to_device(case.x, DEV), to_device(case.logits, DEV)
        mode_out = torch.zeros(1, dtype=torch.int32, device=DEV)
        plan += [
            ("dedup n=%d" % n, n, lambda b, x=x, lg=lg, n=n:
                verify_layer(layer, b, x, lg, n, L.MOE_MODE_DEDUP)),
            ("perslot n=%d" % n, n, lambda b, x=x, lg=lg, n=n:
                verify_layer(layer, b, x, lg, n, L.MOE_MODE_PERSLOT)),
            ("budget n=%d" % n, n, lambda b, x=x, lg=lg, n=n:
                verify_layer_budget(layer, b, x, lg, n, 3, True)),
            ("auto n=%d" % n, n, lambda b, x=x, lg=lg, n=n, mo=mode_out:
                verify_layer_auto(layer, b, x, lg, n, r_auto, mo)),
        ]
    # eager references, each on its own buffers
    ref, bufs = {}, {}
    for name, n, call in plan:
        bufs[name] = VerifyBuffers(layer, n, DEV)
        _clear(bufs[name])
        call(bufs[name])
        torch.cuda.synchronize()
        assert L.moe_get_error(bufs[name].ws) == L.MOE_OK, name
        ref[name] = _snapshot(bufs[name], n)

    # one graph holding every pass, on the same buffers and workspaces
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for name, n, call in plan:
                call(bufs[name])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other = VerifyBuffers(layer, 8, DEV)
    case = make_case(GRAPH_BF16, 8, None, seed=99)
    ox, olg = to_device(case.x, DEV), to_device(case.logits, DEV)
    for rep in range(4):
        print("replay %d" % rep, flush=True)
        for name, _, _ in plan:
            _clear(bufs[name])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, n, _ in plan:
            assert L.moe_get_error(bufs[name].ws) == L.MOE_OK, (rep, name)
            got = _snapshot(bufs[name], n)
            for key, want in ref[name].items():
                assert np.array_equal(got[key], want), (rep, name, key)
        # the program's own eager work between replays, on other buffers
        verify_layer(layer, other, ox, olg, 8, L.MOE_MODE_DEDUP)
        torch.cuda.synchronize()
        assert L.moe_get_error(other.ws) == L.MOE_OK
    del graph
