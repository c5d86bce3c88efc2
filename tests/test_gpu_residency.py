"""GPU: the one-launch pass's bounded waits and its grid on a CU-masked stream.

The workgroups of moe_verify_layer wait for one another through flags, so the
grid must fit the CUs the launch may use, and a wait that cannot complete
gives up after a bounded number of polls and records MOE_ERR_TIMEOUT.

- A stream restricted to 64 CUs by a CU mask: the launch sizes its grid to
  those CUs, so every workgroup is resident and the pass gives the same
  outputs, bit for bit, as on an unrestricted stream (each output row is
  computed by one wavefront in the same order whatever the grid).  The
  workspace's spin word bounds every wait to 2^16 polls here, so a grid that
  did not fit would end in a time-out, not a long wait.
- The time-out path, forced from the host: the workspace's spin word set to
  one poll makes the waits give up (the DOWN phase waits for UP work of other
  workgroups, the combine for every workgroup's DOWN range); the kernel still
  exits normally, the error word reads MOE_ERR_TIMEOUT, and the next call
  with the default limit gives the reference outputs again.
"""
import ctypes as C

import numpy as np
import pytest
import torch

from synth import make_case
from synth.configs import OLMOE

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from moe_speculative_decoding_amd import _lib as L  # noqa: E402
from moe_speculative_decoding_amd.layer import (  # noqa: E402
    DeviceLayer, VerifyBuffers, to_device, verify_layer)
from synth.gen import device_layer_weights  # noqa: E402
from gpu_harness import DEV, _bits  # noqa: E402

SPIN_OFFSET = 192  # byte offset of the spin word in the workspace control block


def _hip():
    """The HIP runtime this process already loaded (the one torch and the
    library use), for the CU-mask stream calls torch does not expose."""
    with open("/proc/self/maps") as fh:
        paths = sorted({ln.split()[-1] for ln in fh if "libamdhip64.so" in ln})
    hip = C.CDLL(paths[0])
    hip.hipExtStreamCreateWithCUMask.argtypes = [C.POINTER(C.c_void_p), C.c_uint32,
                                                 C.POINTER(C.c_uint32)]
    hip.hipExtStreamGetCUMask.argtypes = [C.c_void_p, C.c_uint32, C.POINTER(C.c_uint32)]
    hip.hipStreamSynchronize.argtypes = [C.c_void_p]
    hip.hipStreamDestroy.argtypes = [C.c_void_p]
    return hip


@pytest.fixture(scope="module")
def olmoe_layer():
    w = device_layer_weights(OLMOE, seed=0, layer=0, device=DEV)
    layer = DeviceLayer(OLMOE.E, OLMOE.K, OLMOE.d, OLMOE.f, OLMOE.S, OLMOE.w_dtype,
                        OLMOE.x_dtype, w)
    case = make_case(OLMOE, 8, "markov:0.5", seed=0)
    return layer, to_device(case.x, DEV), to_device(case.logits, DEV)


def _set_spin(buf, polls):
    buf.ws[SPIN_OFFSET:SPIN_OFFSET + 4].view(torch.int32).fill_(polls)


def _reference(layer, x, lg, n):
    ref = VerifyBuffers(layer, n, DEV)
    verify_layer(layer, ref, x, lg, n, L.MOE_MODE_DEDUP)
    torch.cuda.synchronize()
    assert L.moe_get_error(ref.ws) == L.MOE_OK
    return ref


def test_grid_fits_a_cu_masked_stream(olmoe_layer):
    layer, x, lg = olmoe_layer
    n = 8
    ref = _reference(layer, x, lg, n)
    hip = _hip()
    words = 32
    mask = (C.c_uint32 * words)(*([0xFFFFFFFF, 0xFFFFFFFF] + [0] * (words - 2)))
    stream = C.c_void_p()
    assert hip.hipExtStreamCreateWithCUMask(C.byref(stream), words, mask) == 0
    try:
        back = (C.c_uint32 * words)()
        assert hip.hipExtStreamGetCUMask(stream, words, back) == 0
        assert sum(bin(v).count("1") for v in back) == 64
        buf = VerifyBuffers(layer, n, DEV)
        _set_spin(buf, 1 << 16)
        torch.cuda.synchronize()
        print("one-launch pass on a 64-CU stream", flush=True)
        for call in range(2):
            buf.out.zero_()
            torch.cuda.synchronize()
            verify_layer(layer, buf, x, lg, n, L.MOE_MODE_DEDUP, stream=stream.value)
            assert hip.hipStreamSynchronize(stream) == 0
            assert L.moe_get_error(buf.ws, stream.value) == L.MOE_OK, "call %d timed out" % call
            for name in ("out", "y_slots", "U", "union_ids", "offsets", "perm", "bytes"):
                assert np.array_equal(_bits(getattr(buf, name)), _bits(getattr(ref, name))), name
    finally:
        hip.hipStreamDestroy(stream)


def test_bounded_wait_gives_up_and_recovers(olmoe_layer):
    layer, x, lg = olmoe_layer
    n = 8
    ref = _reference(layer, x, lg, n)
    buf = VerifyBuffers(layer, n, DEV)
    _set_spin(buf, 1)
    torch.cuda.synchronize()
    print("one-launch pass with one poll per wait", flush=True)
    verify_layer(layer, buf, x, lg, n, L.MOE_MODE_DEDUP)
    torch.cuda.synchronize()
    assert L.moe_get_error(buf.ws) == L.MOE_ERR_TIMEOUT
    assert L.moe_get_error(buf.ws) == L.MOE_OK  # read and cleared
    _set_spin(buf, 0)  # the default limit
    torch.cuda.synchronize()
    buf.out.zero_()
    verify_layer(layer, buf, x, lg, n, L.MOE_MODE_DEDUP)
    torch.cuda.synchronize()
    assert L.moe_get_error(buf.ws) == L.MOE_OK
    for name in ("out", "y_slots", "bytes"):
        assert np.array_equal(_bits(getattr(buf, name)), _bits(getattr(ref, name))), name
