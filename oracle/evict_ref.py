"""Plain CPU reference of EVICT's utility-guided tree truncation.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/ and
nothing on the product path.  Shares no code with the HIP library.

"Making Every Verified Token Count: Adaptive Verification for MoE Speculative
Decoding", Sec. 3:

* Eq. (7): Score(v) = product of the draft probabilities q(u) over the path
  from the root's child to v;
* Sec. 3.2.1: the top-k nodes by score form the truncated tree T_k (a child's
  score never exceeds its parent's, so T_k is ancestor-closed);
* Eq. (8): the estimated accepted length of T_k is the sum of its scores;
* Eqs. (9)-(10): k* = argmax over 1 <= k <= N of E_hat(T_k) / C(k), with C(k)
  the profiled latency of a step that verifies k nodes (Sec. 3.2.3: prefix
  sums of the sorted scores, divided by the cost table, then an argmax).

Readings (the page leaves them open): the tree is given by parent indices with
parent(v) < v (nodes in breadth-first order; -1 = a child of the root token,
which the target has already sampled); scores are float64 products taken from
the root outward; equal scores rank the lower node index first (a parent
before its child when q = 1, which keeps every T_k ancestor-closed); equal
utilities give the smaller k.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np


def path_scores(parent: Sequence[int], q: Sequence[float]) -> np.ndarray:
    """Eq. (7), root outward: Score(v) = Score(parent(v)) * q(v), Score(root) = 1."""
    n = len(parent)
    s = np.zeros(n, dtype=np.float64)
    for v in range(n):
        p = int(parent[v])
        base = 1.0 if p < 0 else s[p]
        s[v] = base * float(np.float32(q[v]))
    return s


def rank_nodes(scores: np.ndarray) -> List[int]:
    """Sec. 3.2.1: nodes by score, descending; equal scores: lower index first."""
    return sorted(range(len(scores)), key=lambda v: (-scores[v], v))


def evict_select(parent: Sequence[int], q: Sequence[float], cost: Sequence[float]) -> Dict[str, object]:
    s = path_scores(parent, q)
    order = rank_nodes(s)
    expected = np.cumsum([s[v] for v in order])          # Eq. (8) for k = 1..N
    c = np.asarray([float(np.float32(x)) for x in cost], dtype=np.float64)
    utility = expected / c                                # Eq. (9) up to the constant C_AR
    k_best = int(np.argmax(utility)) + 1                  # Eq. (10); first maximum = smallest k
    return {"scores": s, "order": order, "expected": expected, "utility": utility,
            "k_best": k_best}


def is_ancestor_closed(parent: Sequence[int], nodes: Sequence[int]) -> bool:
    chosen = set(int(v) for v in nodes)
    return all(int(parent[v]) < 0 or int(parent[v]) in chosen for v in chosen)
