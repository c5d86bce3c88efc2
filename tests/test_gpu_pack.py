"""GPU: moe_pack_weights, the one-time transform from the SwiGLU matrices as
stored row by row (W_gate, W_up [E][d][f], W_down [E][f][d], fp8 block
scales on the same block grid) to the library's layouts (one row per output
feature).

A layout transform copies bytes: every element and every block scale must
land at its transposed position bit for bit (checked against numpy's
transpose of the same bytes, with ragged tile edges), and a layer packed
from the row-by-row layout must give exactly the verify pass of the same
layer uploaded in the library's layout.
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
    DeviceLayer, VerifyBuffers, to_device, verify_layer)
from gpu_harness import DEV, _bits, upload_layer  # noqa: E402

NP = {"f32": np.uint32, "bf16": np.uint16, "fp8_e4m3": np.uint8}


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(DEV)


def _host(t, dtype):
    return t.cpu().numpy().view(dtype)


@pytest.mark.parametrize("w_dtype,d,f,count", [
    ("f32", 68, 132, 3), ("bf16", 264, 136, 5), ("fp8_e4m3", 384, 256, 2),
    ("fp8_e4m3", 7168, 2048, 1), ("bf16", 2048, 1024, 2),
])
def test_pack_is_a_bitwise_transpose(w_dtype, d, f, count):
    g = np.random.default_rng(d * 31 + f)
    et = NP[w_dtype]
    shape = L.make_shape(8, 2, d, f, 0, w_dtype, "f32" if w_dtype == "f32" else "bf16")
    bits = np.iinfo(et).max + 1
    src = {"gate": g.integers(0, bits, (count, d, f), dtype=np.uint64).astype(et),
           "up": g.integers(0, bits, (count, d, f), dtype=np.uint64).astype(et),
           "down": g.integers(0, bits, (count, f, d), dtype=np.uint64).astype(et)}
    fp8 = w_dtype == "fp8_e4m3"
    ssrc = {}
    if fp8:
        ssrc = {"gate": g.random((count, d // 128, f // 128), dtype=np.float32),
                "up": g.random((count, d // 128, f // 128), dtype=np.float32),
                "down": g.random((count, f // 128, d // 128), dtype=np.float32)}
    dsrc = {k: _dev(v) for k, v in src.items()}
    ddst = {k: torch.full_like(v, 7) for k, v in dsrc.items()}
    dssrc = {k: _dev(v) for k, v in ssrc.items()}
    dsdst = {k: torch.full_like(v, -1.0) for k, v in dssrc.items()}
    print("pack %s d=%d f=%d count=%d" % (w_dtype, d, f, count), flush=True)
    L.moe_pack_weights(shape, count, dsrc["gate"], dsrc["up"], dsrc["down"], dssrc.get("gate"),
                       dssrc.get("up"), dssrc.get("down"), ddst["gate"], ddst["up"],
                       ddst["down"], dsdst.get("gate"), dsdst.get("up"), dsdst.get("down"))
    torch.cuda.synchronize()
    for k in ("gate", "up", "down"):
        want = np.swapaxes(src[k], 1, 2)  # the destination holds [count][cols][rows]
        got = _host(ddst[k], et).reshape(want.shape)
        assert np.array_equal(got, want), k
        if fp8:
            swant = np.swapaxes(ssrc[k], 1, 2)
            sgot = dsdst[k].cpu().numpy().view(np.uint32).reshape(swant.shape)
            assert np.array_equal(sgot, swant.view(np.uint32)), "scales " + k


def test_packed_layer_gives_the_same_pass():
    cfg = LayerConfig(name="pack_fp8", cfg_id=89, E=16, K=4, d=384, f=256, S=1,
                      w_dtype="fp8_e4m3", x_dtype="bf16", n_values=(6,),
                      routing=("markov:0.5",), tolerance=3e-2)
    n = 6
    case = make_case(cfg, n, "markov:0.5", seed=5)
    direct = upload_layer(case)
    # the same experts in the row-by-row layout, packed on the device
    packed = {}
    for group, count in (("routed", cfg.E), ("shared", cfg.S)):
        src = direct.routed if group == "routed" else direct.shared
        rows = {k: torch.from_numpy(np.ascontiguousarray(np.swapaxes(
            src[k].cpu().numpy(), 1, 2))).to(DEV) for k in src}
        dst = {k: torch.empty_like(src[k]) for k in src}
        L.moe_pack_weights(direct.shape, count, rows["w_gate"], rows["w_up"], rows["w_down"],
                           rows["s_gate"], rows["s_up"], rows["s_down"], dst["w_gate"],
                           dst["w_up"], dst["w_down"], dst["s_gate"], dst["s_up"], dst["s_down"])
        packed[group] = dst
    torch.cuda.synchronize()
    layer = DeviceLayer(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype, cfg.x_dtype,
                        packed["routed"], packed["shared"])
    x, lg = to_device(case.x, DEV), to_device(case.logits, DEV)
    outs = []
    for lay in (direct, layer):
        buf = VerifyBuffers(lay, n, DEV)
        verify_layer(lay, buf, x, lg, n, L.MOE_MODE_DEDUP)
        torch.cuda.synchronize()
        assert L.moe_get_error(buf.ws) == L.MOE_OK
        outs.append(buf)
    for name in ("out", "y_slots", "y_shared", "bytes"):
        assert np.array_equal(_bits(getattr(outs[0], name)), _bits(getattr(outs[1], name))), name
