"""Plain CPU reference of a per-layer expert budget on a verify pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/ and
nothing on the product path.  Shares no code with the HIP library.

"MoE-Spec: Expert Budgeting for Efficient Speculative Decoding" (abstract):
every layer of a verification pass loads at most a fixed number C of experts,
the ones that contribute most to the verified tokens, and drops the long tail
of rarely used experts.  The page gives no formula; the readings taken here
(also listed in the design notes):

* an expert's contribution is the sum of the gates of the slots routed to it
  over the pass's n tokens (its share of the combine's weight);
* the C experts of largest contribution are kept; equal contributions go to
  the lower expert id, a NaN contribution ranks below every number, and
  -0.0 equals +0.0 (the same order as the router's top-K);
* the contribution is the plain sum of those gates in float64, slot by slot
  in ascending slot order (the gates are the oracle's own float64 softmax
  values, or the float64 values of gates the caller gives);
* a dropped slot contributes nothing to the layer output (its gate becomes 0
  and its expert output row is zero); with ``renorm`` the kept gates of a
  token that lost a slot are divided by their sum (a token with no kept
  expert keeps gate 0 everywhere; a token that lost nothing is unchanged);
* C >= U leaves the pass unchanged; the union bytes become (min(U, C) + S) b.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np


def _order_key(score: float, e: int):
    # larger score first; NaN after every number; equal scores: lower id first
    v = float(score)
    if math.isnan(v):
        return (1, 0.0, e)
    return (0, -v, e)


def expert_scores(union: Dict[str, object], gates: np.ndarray) -> np.ndarray:
    """Contribution of each union expert: float64 sum of its slots' gates, ascending slot."""
    U = int(union["U"])
    flat = np.asarray(gates, dtype=np.float64).reshape(-1)
    offsets = union["offsets"]
    perm = union["perm"]
    scores = np.zeros(U, dtype=np.float64)
    for u in range(U):
        acc = 0.0
        slots = sorted(int(perm[p]) for p in range(int(offsets[u]), int(offsets[u + 1])))
        for s in slots:
            acc += float(flat[s])
        scores[u] = acc
    return scores


def kept_experts(union: Dict[str, object], scores: np.ndarray, C: int) -> List[int]:
    """Ids of the (at most) C union experts of largest contribution, ascending."""
    U = int(union["U"])
    ids = [int(union["union_ids"][u]) for u in range(U)]
    order = sorted(range(U), key=lambda u: _order_key(scores[u], ids[u]))
    return sorted(ids[u] for u in order[:C])


def apply_budget(ids: np.ndarray, gates: np.ndarray, union: Dict[str, object], C: int,
                 renorm: bool = False) -> Dict[str, object]:
    """The budgeted union and gates of one pass.

    ``union`` is the plain union of ``ids`` (``build_union``); ``gates`` the
    pass's gates [n][K].  Returns a union dictionary of the same form, whose
    groups are the kept experts only (offsets from U on hold the number of
    kept slots; perm lists the kept slots grouped by expert, then the dropped
    slots in ascending order; slot_rank is -1 for a dropped slot), plus
    ``gates`` float64 [n][K] (dropped slots 0, kept ones renormalised per token
    when ``renorm`` and the token lost a slot) and ``kept`` (the kept expert
    ids).
    """
    ids = np.asarray(ids)
    n, K = ids.shape
    nk = n * K
    U = int(union["U"])
    g64 = np.asarray(gates, dtype=np.float64)
    scores = expert_scores(union, g64)
    kept = kept_experts(union, scores, C)
    keep = set(kept)
    flat = [int(v) for v in ids.reshape(-1)]
    cap = len(union["union_ids"])
    Uk = len(kept)
    union_ids = np.full(cap, -1, dtype=np.int32)
    union_ids[:Uk] = kept
    position = {e: u for u, e in enumerate(kept)}
    kept_slots = sorted((s for s in range(nk) if flat[s] in keep), key=lambda s: (flat[s], s))
    dropped_slots = [s for s in range(nk) if flat[s] not in keep]
    offsets = np.full(cap + 1, len(kept_slots), dtype=np.int32)
    run = 0
    for u, e in enumerate(kept):
        offsets[u] = run
        run += sum(1 for s in kept_slots if flat[s] == e)
    perm = np.array(kept_slots + dropped_slots, dtype=np.int32)
    slot_rank = np.array([position.get(v, -1) for v in flat], dtype=np.int32)
    g = np.zeros((n, K))
    for t in range(n):
        total = 0.0
        lost = False
        for k in range(K):
            if flat[t * K + k] in keep:
                g[t, k] = g64[t, k]
                total += g64[t, k]
            else:
                lost = True
        if renorm and lost and total > 0.0:
            g[t] /= total
    return {"U": Uk, "union_ids": union_ids, "offsets": offsets, "perm": perm,
            "slot_rank": slot_rank, "gates": g, "kept": kept, "scores": scores,
            "U_before": U}


def verify_op_budget(case, C: int, renorm: bool = False,
                     ids: Optional[np.ndarray] = None,
                     gates: Optional[np.ndarray] = None) -> Dict[str, object]:
    """Route, union, budget, deduplicating FFN over the kept experts and combine."""
    from .moe_ref import build_union, byte_counts, combine, ffn_dedup, route_topk

    cfg = case.cfg
    if ids is None:
        ids, gates = route_topk(case.logits, cfg.K)
    un = build_union(ids, cfg.E)
    bud = apply_budget(ids, gates, un, C, renorm)
    y, ysh, read = ffn_dedup(case.x, ids, bud, case.expert, case.shared, cfg.S,
                             cfg.w_dtype, cfg.x_dtype, cfg.d, cfg.f)
    # dropped slots were never computed: their rows stay zero
    out = combine(y, bud["gates"], ysh if cfg.S else None)
    ub, rb = byte_counts(cfg.d, cfg.f, cfg.w_dtype, cfg.K, cfg.S, case.n, int(bud["U"]))
    return {"ids": ids, "gates": bud["gates"], "union": bud, "y_slots": y, "y_shared": ysh,
            "out": out, "bytes_read": read, "union_bytes": ub, "requested_bytes": rb}
