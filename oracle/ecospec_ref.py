"""Plain CPU reference of EcoSpec's cost-aware draft selection.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/ and
nothing on the product path.  Shares no code with the HIP library.

"Less Experts, Faster Decoding: Cost-Aware Speculative Decoding for
Mixture-of-Experts", Sec. 4.2 and Algorithm 1:

* Eq. (7): the path footprint E_traj(t) is the union of the predicted
  (layer, expert) sets of the nodes on the path from the root to t;
* Eq. (8): the marginal cost of t under the buffer B is |E_traj(t) \\ B|;
* Eq. (9): Score(t) = P(t) / (cost + eps), P(t) the cumulative draft
  probability of the path;
* Algorithm 1: while fewer than gamma nodes are selected, score every
  unselected node, select the best, and add its footprint to B.

Readings: the tree is given by parent indices with parent(t) < t (-1 for the
root token(s)); P is the float64 product of the draft probabilities from the
root outward; equal scores select the lower node index (a parent before its
child, so the selection stays prefix-closed, Sec. 4.2 "Prefix Consistency");
(layer, expert) sets are Python sets of pairs here.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np


def cumulative_probability(parent: Sequence[int], q: Sequence[float]) -> np.ndarray:
    n = len(parent)
    P = np.zeros(n, dtype=np.float64)
    for t in range(n):
        p = int(parent[t])
        P[t] = (1.0 if p < 0 else P[p]) * float(np.float32(q[t]))
    return P


def path_footprints(parent: Sequence[int], pred: Sequence[set]) -> List[set]:
    """Eq. (7) as Python sets of (layer, expert) pairs."""
    out: List[set] = []
    for t in range(len(parent)):
        p = int(parent[t])
        out.append(set(pred[t]) | (out[p] if p >= 0 else set()))
    return out


def ecospec_select(parent: Sequence[int], q: Sequence[float], pred: Sequence[set], gamma: int,
                   eps: float, buffer0: Optional[set] = None) -> Dict[str, object]:
    """Algorithm 1 with sets: returns the selected nodes in selection order,
    the scores seen at each step and the final buffer."""
    P = cumulative_probability(parent, q)
    traj = path_footprints(parent, pred)
    B = set(buffer0 or ())
    selected: List[int] = []
    steps = []
    while len(selected) < min(gamma, len(parent)):
        scores = {}
        for t in range(len(parent)):
            if t in selected:
                continue
            cost = len(traj[t] - B)
            scores[t] = P[t] / (cost + eps)
        best = max(scores, key=lambda t: (scores[t], -t))
        steps.append(scores)
        selected.append(best)
        B |= traj[best]
    return {"selected": selected, "P": P, "steps": steps, "buffer": B}
