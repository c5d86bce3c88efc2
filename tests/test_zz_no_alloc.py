"""GPU: moe_verify_layer_noalloc (the one-launch pass on the library's static
scratch) against moe_verify_layer on a caller-allocated workspace.

Both run the same kernels, so every output must agree bit for bit.  The
calls run back to back on one GPU, so the second call finds the scratch as
the first left it: the first pass is the larger one (n = 8, slot outputs in
the scratch), the next ones smaller, in both modes, with bf16 weights and a
shared expert (slot and shared outputs in the scratch) and with fp8 weights.
The layer output of the first pass is also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import make_case
from synth.configs import LayerConfig

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from moe_speculative_decoding_amd import _lib as L  # noqa: E402
from moe_speculative_decoding_amd.layer import VerifyBuffers, to_device, verify_layer  # noqa: E402
from gpu_harness import DEV, _bits, check_vectors, upload_layer  # noqa: E402

NOALLOC_BF16 = LayerConfig(name="noalloc_bf16", cfg_id=86, E=24, K=4, d=264, f=136, S=1,
                           w_dtype="bf16", x_dtype="bf16", n_values=(8, 3),
                           routing=("markov:0.5",), tolerance=1e-2)
NOALLOC_FP8 = LayerConfig(name="noalloc_fp8", cfg_id=87, E=16, K=4, d=384, f=256, S=0,
                          w_dtype="fp8_e4m3", x_dtype="bf16", n_values=(5, 2),
                          routing=("markov:0.5",), tolerance=3e-2)

_UNION = ("U", "union_ids", "offsets", "perm", "slot_rank")


def _fresh(layer, n):
    buf = VerifyBuffers(layer, n, DEV)
    for t in (buf.out, buf.y_slots, buf.y_shared, buf.ids, buf.gates, buf.bytes) + \
            tuple(getattr(buf, k) for k in _UNION):
        t.fill_(-1)  # a fill kernel: anything the call leaves unwritten shows
    return buf


def _with_ws(layer, buf, x, lg, n, mode, keep):
    """moe_verify_layer with the same outputs as _noalloc asks for"""
    if keep:
        verify_layer(layer, buf, x, lg, n, mode)
    else:
        L.moe_verify_layer(layer.shape, layer.weights, lg, x, n, mode, buf.out, buf.out_dtype,
                           bytes_=buf.bytes, ws=buf.ws, ws_bytes=buf.ws_bytes)


def _noalloc(layer, buf, x, lg, n, mode, keep):
    ysh = buf.y_shared if layer.S > 0 else None
    if keep:
        L.moe_verify_layer_noalloc(layer.shape, layer.weights, lg, x, n, mode, buf.out,
                                   buf.out_dtype, buf.ids, buf.gates, buf.U, buf.union_ids,
                                   buf.offsets, buf.perm, buf.slot_rank, buf.y_slots, ysh,
                                   buf.bytes)
    else:
        L.moe_verify_layer_noalloc(layer.shape, layer.weights, lg, x, n, mode, buf.out,
                                   buf.out_dtype, bytes_=buf.bytes)


@pytest.mark.parametrize("cfg", [NOALLOC_BF16, NOALLOC_FP8], ids=lambda c: c.name)
def test_noalloc_matches_workspace_pass(cfg):
    big_n, small_n = cfg.n_values
    case0 = make_case(cfg, big_n, "markov:0.5", seed=3)
    layer = upload_layer(case0)  # every expert of the layer
    # (n, mode, keep outputs): the first call is the largest; y_slots in the
    # scratch (keep = False) on the first, caller's arrays on a later one
    plan = [(big_n, L.MOE_MODE_DEDUP, False), (small_n, L.MOE_MODE_PERSLOT, False),
            (small_n, L.MOE_MODE_DEDUP, True), (big_n, L.MOE_MODE_PERSLOT, True)]
    for i, (n, mode, keep) in enumerate(plan):
        case = case0 if i == 0 else make_case(cfg, n, "markov:0.5", seed=10 + i)
        x, lg = to_device(case.x, DEV), to_device(case.logits, DEV)
        print("noalloc %s call %d: n=%d mode=%d keep=%d" % (cfg.name, i, n, mode, keep), flush=True)
        ref = _fresh(layer, n)
        _with_ws(layer, ref, x, lg, n, mode, keep)
        got = _fresh(layer, n)
        _noalloc(layer, got, x, lg, n, mode, keep)
        torch.cuda.synchronize()
        assert L.moe_get_error(ref.ws) == L.MOE_OK
        assert L.moe_get_error(None) == L.MOE_OK
        names = ["out", "bytes"] + (["y_slots", "ids", "gates"] if keep else [])
        if keep and layer.S:
            names.append("y_shared")
        if keep and mode == L.MOE_MODE_DEDUP:
            names += list(_UNION)
        for name in names:
            a, b = getattr(got, name), getattr(ref, name)
            if name in ("out", "y_slots", "ids", "gates", "y_shared"):
                a, b = a[:n], b[:n]
            assert np.array_equal(_bits(a), _bits(b)), "call %d: %s differs" % (i, name)
        if i == 0:
            r = oracle.verify_op(case, "dedup")
            check_vectors(got.out[:n].float().cpu().numpy(), r["out"], cfg.tolerance, "out")


def test_noalloc_rejects_passes_beyond_the_scratch():
    # n*K*d*4 B of slot outputs kept in the scratch exceed its 16 MiB; nothing
    # is enqueued (the check runs on the host before any launch)
    big = LayerConfig(name="noalloc_big", cfg_id=88, E=16, K=8, d=16384, f=128, S=0,
                      w_dtype="bf16", x_dtype="bf16", n_values=(32,), routing=("iid",),
                      tolerance=1e-2)
    shape = L.make_shape(big.E, big.K, big.d, big.f, big.S, big.w_dtype, big.x_dtype)
    w = torch.zeros(16, dtype=torch.uint8, device=DEV)
    weights = L.make_weights(w_gate=w, w_up=w, w_down=w)
    lg = torch.zeros(32, big.E, dtype=torch.float32, device=DEV)
    x = torch.zeros(32, big.d, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(32, big.d, dtype=torch.float32, device=DEV)
    with pytest.raises(L.MoeError) as ei:
        L.moe_verify_layer_noalloc(shape, weights, lg, x, 32, L.MOE_MODE_DEDUP, out, L.MOE_F32)
    assert ei.value.status == L.MOE_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert L.moe_get_error(None) == L.MOE_OK
