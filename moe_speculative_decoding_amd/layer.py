"""Device buffers of one MoE layer and the chain of entry points of one verify pass.

Only allocation (torch, on the GPU) and calls through the C ABI happen here;
every step of the pass runs in the HIP library.  The calls are asynchronous:
an argument error raises at once, but what the device detects (expert ids out
of range, a hand-over wait that gave up) lands in the workspace's error word,
which `_lib.moe_get_error(buf.ws)` reads after synchronising.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import _lib as L

ROUTED = ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """Upload a host array bit-for-bit (uint16 bf16 patterns travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceLayer:
    """Expert weights of one layer on the device, in the ABI layouts."""

    def __init__(self, E: int, K: int, d: int, f: int, S: int, w_dtype: str, x_dtype: str,
                 routed: Dict[str, torch.Tensor], shared: Optional[Dict[str, torch.Tensor]] = None):
        self.E, self.K, self.d, self.f, self.S = E, K, d, f, S
        self.w_dtype, self.x_dtype = w_dtype, x_dtype
        self.shape = L.make_shape(E, K, d, f, S, w_dtype, x_dtype)
        self.routed = routed
        self.shared = shared or {}
        kw = {k: routed.get(k) for k in ROUTED}
        for k in ROUTED:  # w_gate -> sh_gate, s_gate -> sh_s_gate
            kw["sh_" + (k[2:] if k.startswith("w_") else k)] = self.shared.get(k)
        self.weights = L.make_weights(**kw)

    @classmethod
    def from_arrays(cls, cfg, routed: Dict[str, np.ndarray], shared: Optional[Dict[str, np.ndarray]],
                    device) -> "DeviceLayer":
        r = {k: to_device(v, device) for k, v in routed.items()}
        s = {k: to_device(v, device) for k, v in shared.items()} if shared else None
        return cls(cfg.E, cfg.K, cfg.d, cfg.f, cfg.S, cfg.w_dtype, cfg.x_dtype, r, s)

    def expert_bytes(self) -> int:
        ub, _ = L.moe_byte_counts(self.shape, 1, self.K)
        return ub // (self.K + self.S)


class VerifyBuffers:
    """Every device array one verify pass of up to n_max tokens writes."""

    def __init__(self, layer: DeviceLayer, n_max: int, device, out_dtype: int = L.MOE_F32):
        E, K, d, S = layer.E, layer.K, layer.d, layer.S
        i32 = dict(dtype=torch.int32, device=device)
        cap = min(n_max * K, E)
        self.n_max = n_max
        self.ids = torch.zeros(n_max, K, **i32)
        self.gates = torch.zeros(n_max, K, dtype=torch.float32, device=device)
        self.U = torch.zeros(1, **i32)
        self.union_ids = torch.zeros(cap, **i32)
        self.offsets = torch.zeros(cap + 1, **i32)
        self.perm = torch.zeros(n_max * K, **i32)
        self.slot_rank = torch.zeros(n_max * K, **i32)
        self.y_slots = torch.zeros(n_max, K, d, dtype=torch.float32, device=device)
        self.y_shared = torch.zeros(n_max, max(S, 1), d, dtype=torch.float32, device=device)
        self.out_dtype = out_dtype
        self.out = torch.zeros(n_max, d, dtype=torch.float32 if out_dtype == L.MOE_F32
                               else torch.bfloat16, device=device)
        self.bytes = torch.zeros(2, dtype=torch.int64, device=device)
        self.ws_bytes = max(L.moe_workspace_size(layer.shape, n_max, L.MOE_MODE_DEDUP),
                            L.moe_workspace_size(layer.shape, n_max, L.MOE_MODE_PERSLOT))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        L.moe_workspace_init(self.ws, self.ws_bytes)


def verify_pass(layer: DeviceLayer, buf: VerifyBuffers, x: torch.Tensor, logits: torch.Tensor,
                n: int, mode: int = L.MOE_MODE_DEDUP, stream=None) -> None:
    """route -> (union) -> expert FFN -> combine, all enqueued on one stream."""
    K, E, S, d = layer.K, layer.E, layer.S, layer.d
    ysh = buf.y_shared if S > 0 else None
    if mode == L.MOE_MODE_DEDUP:
        L.moe_route_union(logits, n, E, K, buf.ids, buf.gates, buf.U, buf.union_ids, buf.offsets,
                          buf.perm, buf.slot_rank, stream)
        L.moe_expert_ffn_dedup(layer.shape, layer.weights, x, n, buf.U, buf.union_ids, buf.offsets,
                               buf.perm, buf.y_slots, ysh, buf.bytes, buf.ws, buf.ws_bytes, stream)
    else:
        L.moe_route_topk(logits, n, E, K, buf.ids, buf.gates, stream)
        L.moe_expert_ffn_perslot(layer.shape, layer.weights, x, n, buf.ids, buf.y_slots, ysh,
                                 buf.bytes, buf.ws, buf.ws_bytes, stream)
    L.moe_combine(buf.y_slots, buf.gates, ysh, n, K, S, d, buf.out, buf.out_dtype, stream)


def verify_layer(layer: DeviceLayer, buf: VerifyBuffers, x: torch.Tensor, logits: torch.Tensor,
                 n: int, mode: int = L.MOE_MODE_DEDUP, stream=None, keep: bool = True) -> None:
    """The same pass in one launch (moe_verify_layer).  keep=False leaves the
    routing, union and slot outputs to the workspace and writes only out."""
    ysh = buf.y_shared if layer.S > 0 else None
    if keep:
        L.moe_verify_layer(layer.shape, layer.weights, logits, x, n, mode, buf.out, buf.out_dtype,
                           buf.ids, buf.gates, buf.U, buf.union_ids, buf.offsets, buf.perm,
                           buf.slot_rank, buf.y_slots, ysh, buf.bytes, buf.ws, buf.ws_bytes,
                           stream)
    else:
        L.moe_verify_layer(layer.shape, layer.weights, logits, x, n, mode, buf.out, buf.out_dtype,
                           ws=buf.ws, ws_bytes=buf.ws_bytes, stream=stream)


def verify_layer_auto(layer: DeviceLayer, buf: VerifyBuffers, x: torch.Tensor,
                      logits: torch.Tensor, n: int, r: float, mode_out: torch.Tensor,
                      stream=None) -> None:
    """The one-launch pass with the mode chosen on the device from the pass's
    own union and the measured bandwidth ratio r (moe_verify_layer_auto)."""
    L.moe_verify_layer_auto(layer.shape, layer.weights, logits, x, n, r, buf.out, buf.out_dtype,
                            mode_out, buf.bytes, buf.ws, buf.ws_bytes, stream)


def verify_pass_budget(layer: DeviceLayer, buf: VerifyBuffers, x: torch.Tensor,
                       logits: torch.Tensor, n: int, C: int, renorm: bool = False,
                       stream=None) -> None:
    """route + union -> expert budget (gates rewritten in place) -> deduplicating
    FFN over the kept experts -> combine, all enqueued on one stream."""
    K, E, S, d = layer.K, layer.E, layer.S, layer.d
    ysh = buf.y_shared if S > 0 else None
    L.moe_route_union(logits, n, E, K, buf.ids, buf.gates, buf.U, buf.union_ids, buf.offsets,
                      buf.perm, buf.slot_rank, stream)
    L.moe_expert_budget(buf.gates, n, K, E, C, renorm, buf.U, buf.union_ids, buf.offsets,
                        buf.perm, buf.slot_rank, buf.gates, stream)
    L.moe_expert_ffn_dedup(layer.shape, layer.weights, x, n, buf.U, buf.union_ids, buf.offsets,
                           buf.perm, buf.y_slots, ysh, buf.bytes, buf.ws, buf.ws_bytes, stream)
    L.moe_combine(buf.y_slots, buf.gates, ysh, n, K, S, d, buf.out, buf.out_dtype, stream)


def verify_layer_budget(layer: DeviceLayer, buf: VerifyBuffers, x: torch.Tensor,
                        logits: torch.Tensor, n: int, C: int, renorm: bool = False,
                        stream=None, keep: bool = True) -> None:
    """The budgeted pass in one launch (moe_verify_layer_budget)."""
    ysh = buf.y_shared if layer.S > 0 else None
    if keep:
        L.moe_verify_layer_budget(layer.shape, layer.weights, logits, x, n, C, renorm, buf.out,
                                  buf.out_dtype, buf.ids, buf.gates, buf.U, buf.union_ids,
                                  buf.offsets, buf.perm, buf.slot_rank, buf.y_slots, ysh,
                                  buf.bytes, buf.ws, buf.ws_bytes, stream)
    else:
        L.moe_verify_layer_budget(layer.shape, layer.weights, logits, x, n, C, renorm, buf.out,
                                  buf.out_dtype, ws=buf.ws, ws_bytes=buf.ws_bytes, stream=stream)
