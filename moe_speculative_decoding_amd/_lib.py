"""ctypes binding of ``libmoe_verify.so`` — argument marshalling only.

Every function here has the name and the parameter order of its C entry
point in ``include/moe_verify.h``; device buffers are passed as torch tensors
(their ``data_ptr()``) or raw integer addresses, and the stream defaults to
torch's current stream.  A non-OK status raises ``MoeError``.  Nothing is
computed in Python, and there is no fallback: without the built library,
importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_VERIFY_LIB may name another build of the same library (same ABI)
LIB_PATH = os.environ.get("MOE_VERIFY_LIB") or os.path.join(_HERE, "libmoe_verify.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE = 0, 1, 2, 3
MOE_ERR_HIP, MOE_ERR_BAD_IDS, MOE_ERR_TIMEOUT, MOE_ERR_BAD_TREE = 4, 5, 6, 7
MOE_ERR_TOO_LARGE = 8
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_MODE_DEDUP, MOE_MODE_PERSLOT = 0, 1

DTYPE_CODES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8_e4m3": MOE_FP8_E4M3}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s: %s (status %d)" % (where, status_str(status), status)
        if status == MOE_ERR_HIP:
            msg += ": hipError %d %s" % (lib.moe_last_hip_error(), lib.moe_hip_error_string().decode())
        super().__init__(msg)


class moe_shape(C.Structure):
    _fields_ = [("E", C.c_int32), ("K", C.c_int32), ("d", C.c_int32), ("f", C.c_int32),
                ("S", C.c_int32), ("w_dtype", C.c_int32), ("x_dtype", C.c_int32)]


class moe_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
        "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down")]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmoe_verify.so is not built (run __graft_entry__.build() or "
                          "python -m moe_speculative_decoding_amd.build): %s" % LIB_PATH)
    return C.CDLL(LIB_PATH)


lib = _load()

_P = C.c_void_p
_I = C.c_int32
_SIG = {
    "moe_route_topk": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_build_union": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_route_union": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_budget": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_dedup": (_I, [C.POINTER(moe_shape), C.POINTER(moe_weights), _P, _I, _P, _P,
                                  _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_expert_ffn_perslot": (_I, [C.POINTER(moe_shape), C.POINTER(moe_weights), _P, _I, _P, _P,
                                    _P, _P, _P, C.c_size_t, _P]),
    "moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _I, _P]),
    "moe_verify_layer": (_I, [C.POINTER(moe_shape), C.POINTER(moe_weights), _P, _P, _I, _I, _P,
                              _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_verify_layer_noalloc": (_I, [C.POINTER(moe_shape), C.POINTER(moe_weights), _P, _P, _I,
                                      _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_verify_layer_budget": (_I, [C.POINTER(moe_shape), C.POINTER(moe_weights), _P, _P, _I,
                                     _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     C.c_size_t, _P]),
    "moe_verify_layer_auto": (_I, [C.POINTER(moe_shape), C.POINTER(moe_weights), _P, _P, _I,
                                   C.c_float, _P, _I, _P, _P, _P, C.c_size_t, _P]),
    "moe_evict_select": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_ecospec_select": (_I, [_P, _P, _P, _P, _I, _I, _I, C.c_double, _P, _P, _P, C.c_size_t,
                                _P]),
    "moe_bellman_policy": (_I, [_P, _P, _I, _I, _P, _P, _P, C.c_size_t, _P]),
    "moe_pack_weights": (_I, [C.POINTER(moe_shape), _I] + [_P] * 12 + [_P]),
    "moe_workspace_size": (C.c_size_t, [C.POINTER(moe_shape), _I, _I]),
    "moe_workspace_init": (_I, [_P, C.c_size_t, _P]),
    "moe_byte_counts": (_I, [C.POINTER(moe_shape), _I, _I, C.POINTER(C.c_uint64),
                             C.POINTER(C.c_uint64)]),
    "moe_get_error": (_I, [_P, _P]),
    "moe_unit_partition": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_decode_fp8": (_I, [_P, _P, C.c_int64, _P]),
    "moe_status_str": (C.c_char_p, [_I]),
    "moe_last_hip_error": (_I, []),
    "moe_hip_error_string": (C.c_char_p, []),
    "moe_abi_version": (_I, []),
}
for _name, (_res, _args) in _SIG.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def status_str(status: int) -> str:
    return lib.moe_status_str(int(status)).decode()


def ptr(t) -> Optional[int]:
    """Device address of a tensor (None/0 stays null; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t or None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def make_shape(E: int, K: int, d: int, f: int, S: int, w_dtype: str, x_dtype: str) -> moe_shape:
    return moe_shape(E, K, d, f, S, DTYPE_CODES[w_dtype], DTYPE_CODES[x_dtype])


def make_weights(**tensors) -> moe_weights:
    w = moe_weights()
    fields = {f[0] for f in moe_weights._fields_}
    for k, v in tensors.items():
        if k not in fields:
            raise KeyError("moe_weights has no field %r" % k)
        setattr(w, k, ptr(v))
    return w


# ---------------------------------------------------------------- entry points
def moe_route_topk(logits, n, E, K, ids, gates, stream=None) -> None:
    _check(lib.moe_route_topk(ptr(logits), n, E, K, ptr(ids), ptr(gates), _stream(stream)),
           "moe_route_topk")


def moe_build_union(ids, n, K, E, U, union_ids, offsets, perm, slot_rank, stream=None) -> None:
    _check(lib.moe_build_union(ptr(ids), n, K, E, ptr(U), ptr(union_ids), ptr(offsets), ptr(perm),
                               ptr(slot_rank), _stream(stream)), "moe_build_union")


def moe_route_union(logits, n, E, K, ids, gates, U, union_ids, offsets, perm, slot_rank,
                    stream=None) -> None:
    _check(lib.moe_route_union(ptr(logits), n, E, K, ptr(ids), ptr(gates), ptr(U), ptr(union_ids),
                               ptr(offsets), ptr(perm), ptr(slot_rank), _stream(stream)),
           "moe_route_union")


def moe_expert_budget(gates, n, K, E, C_, renorm, U, union_ids, offsets, perm, slot_rank,
                      gates_out, stream=None) -> None:
    _check(lib.moe_expert_budget(ptr(gates), n, K, E, C_, int(renorm), ptr(U), ptr(union_ids),
                                 ptr(offsets), ptr(perm), ptr(slot_rank), ptr(gates_out),
                                 _stream(stream)), "moe_expert_budget")


def moe_expert_ffn_dedup(shape: moe_shape, w: moe_weights, x, n, U, union_ids, offsets, perm,
                         y_slots, y_shared, bytes_, ws, ws_bytes, stream=None) -> None:
    _check(lib.moe_expert_ffn_dedup(C.byref(shape), C.byref(w), ptr(x), n, ptr(U), ptr(union_ids),
                                    ptr(offsets), ptr(perm), ptr(y_slots), ptr(y_shared),
                                    ptr(bytes_), ptr(ws), ws_bytes, _stream(stream)),
           "moe_expert_ffn_dedup")


def moe_expert_ffn_perslot(shape: moe_shape, w: moe_weights, x, n, ids, y_slots, y_shared, bytes_,
                           ws, ws_bytes, stream=None) -> None:
    _check(lib.moe_expert_ffn_perslot(C.byref(shape), C.byref(w), ptr(x), n, ptr(ids),
                                      ptr(y_slots), ptr(y_shared), ptr(bytes_), ptr(ws), ws_bytes,
                                      _stream(stream)), "moe_expert_ffn_perslot")


def moe_combine(y_slots, gates, y_shared, n, K, S, d, out, out_dtype, stream=None) -> None:
    _check(lib.moe_combine(ptr(y_slots), ptr(gates), ptr(y_shared), n, K, S, d, ptr(out),
                           out_dtype, _stream(stream)), "moe_combine")


def moe_verify_layer(shape: moe_shape, w: moe_weights, logits, x, n, mode, out, out_dtype,
                     ids=None, gates=None, U=None, union_ids=None, offsets=None, perm=None,
                     slot_rank=None, y_slots=None, y_shared=None, bytes_=None, ws=None,
                     ws_bytes=0, stream=None) -> None:
    _check(lib.moe_verify_layer(C.byref(shape), C.byref(w), ptr(logits), ptr(x), n, mode, ptr(out),
                                out_dtype, ptr(ids), ptr(gates), ptr(U), ptr(union_ids),
                                ptr(offsets), ptr(perm), ptr(slot_rank), ptr(y_slots),
                                ptr(y_shared), ptr(bytes_), ptr(ws), ws_bytes, _stream(stream)),
           "moe_verify_layer")


def moe_verify_layer_noalloc(shape: moe_shape, w: moe_weights, logits, x, n, mode, out,
                             out_dtype, ids=None, gates=None, U=None, union_ids=None,
                             offsets=None, perm=None, slot_rank=None, y_slots=None,
                             y_shared=None, bytes_=None, stream=None) -> None:
    _check(lib.moe_verify_layer_noalloc(C.byref(shape), C.byref(w), ptr(logits), ptr(x), n, mode,
                                        ptr(out), out_dtype, ptr(ids), ptr(gates), ptr(U),
                                        ptr(union_ids), ptr(offsets), ptr(perm), ptr(slot_rank),
                                        ptr(y_slots), ptr(y_shared), ptr(bytes_), _stream(stream)),
           "moe_verify_layer_noalloc")


def moe_verify_layer_budget(shape: moe_shape, w: moe_weights, logits, x, n, C_, renorm, out,
                            out_dtype, ids=None, gates=None, U=None, union_ids=None, offsets=None,
                            perm=None, slot_rank=None, y_slots=None, y_shared=None, bytes_=None,
                            ws=None, ws_bytes=0, stream=None) -> None:
    _check(lib.moe_verify_layer_budget(C.byref(shape), C.byref(w), ptr(logits), ptr(x), n, C_,
                                       int(renorm), ptr(out), out_dtype, ptr(ids), ptr(gates),
                                       ptr(U), ptr(union_ids), ptr(offsets), ptr(perm),
                                       ptr(slot_rank), ptr(y_slots), ptr(y_shared), ptr(bytes_),
                                       ptr(ws), ws_bytes, _stream(stream)),
           "moe_verify_layer_budget")


def moe_verify_layer_auto(shape: moe_shape, w: moe_weights, logits, x, n, r, out, out_dtype,
                          mode_out=None, bytes_=None, ws=None, ws_bytes=0, stream=None) -> None:
    _check(lib.moe_verify_layer_auto(C.byref(shape), C.byref(w), ptr(logits), ptr(x), n, float(r),
                                     ptr(out), out_dtype, ptr(mode_out), ptr(bytes_), ptr(ws),
                                     ws_bytes, _stream(stream)), "moe_verify_layer_auto")


def moe_evict_select(parent, q, cost, N, order, scores, expected, k_best, ws, ws_bytes,
                     stream=None) -> None:
    _check(lib.moe_evict_select(ptr(parent), ptr(q), ptr(cost), N, ptr(order), ptr(scores),
                                ptr(expected), ptr(k_best), ptr(ws), ws_bytes, _stream(stream)),
           "moe_evict_select")


def moe_ecospec_select(parent, q, pred, buffer0, N, W, gamma, eps, selected, buffer_out, ws,
                       ws_bytes, stream=None) -> None:
    _check(lib.moe_ecospec_select(ptr(parent), ptr(q), ptr(pred), ptr(buffer0), N, W, gamma,
                                  float(eps), ptr(selected), ptr(buffer_out), ptr(ws), ws_bytes,
                                  _stream(stream)), "moe_ecospec_select")


def moe_bellman_policy(q, cost, N, L_, dp, k_best, ws, ws_bytes, stream=None) -> None:
    _check(lib.moe_bellman_policy(ptr(q), ptr(cost), N, L_, ptr(dp), ptr(k_best), ptr(ws),
                                  ws_bytes, _stream(stream)), "moe_bellman_policy")


def moe_pack_weights(shape: moe_shape, count, src_gate, src_up, src_down, src_s_gate,
                     src_s_up, src_s_down, dst_gate, dst_up, dst_down, dst_s_gate, dst_s_up,
                     dst_s_down, stream=None) -> None:
    _check(lib.moe_pack_weights(C.byref(shape), count, ptr(src_gate), ptr(src_up), ptr(src_down),
                                ptr(src_s_gate), ptr(src_s_up), ptr(src_s_down), ptr(dst_gate),
                                ptr(dst_up), ptr(dst_down), ptr(dst_s_gate), ptr(dst_s_up),
                                ptr(dst_s_down), _stream(stream)), "moe_pack_weights")


def moe_workspace_size(shape: moe_shape, n_max: int, mode: int) -> int:
    return int(lib.moe_workspace_size(C.byref(shape), n_max, mode))


def moe_workspace_init(ws, ws_bytes, stream=None) -> None:
    _check(lib.moe_workspace_init(ptr(ws), ws_bytes, _stream(stream)), "moe_workspace_init")


def moe_byte_counts(shape: moe_shape, n: int, U: int):
    ub, rb = C.c_uint64(0), C.c_uint64(0)
    _check(lib.moe_byte_counts(C.byref(shape), n, U, C.byref(ub), C.byref(rb)), "moe_byte_counts")
    return int(ub.value), int(rb.value)


def moe_get_error(ws, stream=None) -> int:
    """Status of the device error word (also returned, not raised); ws=None reads
    the error word of moe_verify_layer_noalloc's scratch on the current device."""
    return int(lib.moe_get_error(ptr(ws), _stream(stream)))


def moe_unit_partition(counts, tile: int, up: bool, upg: int, grid: int):
    """The one-launch pass's unit partition of one phase, computed on the host:
    (first_unit [grid + 1], owner_lo [ng], owner_hi [ng]) as numpy arrays."""
    import numpy as np
    cnt = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
    ng = int(cnt.size)
    first = np.zeros(grid + 1, dtype=np.int64)
    lo = np.zeros(max(ng, 1), dtype=np.int32)
    hi = np.zeros(max(ng, 1), dtype=np.int32)
    _check(lib.moe_unit_partition(cnt.ctypes.data, ng, tile, 1 if up else 0, upg, grid,
                                  first.ctypes.data, lo.ctypes.data, hi.ctypes.data),
           "moe_unit_partition")
    return first, lo[:ng], hi[:ng]


def moe_decode_fp8(codes, out, count, stream=None) -> None:
    _check(lib.moe_decode_fp8(ptr(codes), ptr(out), count, _stream(stream)), "moe_decode_fp8")


def moe_abi_version() -> int:
    return int(lib.moe_abi_version())
