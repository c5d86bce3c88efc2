"""Plain CPU reference of the sequence-conditioned Bellman oracle of draft lengths.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/ and
nothing on the product path.  Shares no code with the HIP library.

"The Limits of Speculation: Bounding Speculative Decoding in MoE", Sec. 4:

* Sec. 4.1: the state is the position i in a reference sequence of N tokens
  (N absorbing, dp[N] = 0); the action is a draft length k in 1..L; accepting
  a of the k drafts moves the state to min(i + a + 1, N) (the target always
  adds one token);
* Eq. (7): with p_j the draft model's probability of the (j+1)-th reference
  token of the window, P(a | k) = (prod_{j<a} p_j) (1 - p_a) for a < k and
  P(k | k) = prod_{j<k} p_j;
* Eq. (8): dp[i] = min_k sum_{a=0..k} P(a | k) (Cost(i, k, a) + dp[min(i + a + 1, N)]),
  solved by backward induction from dp[N] = 0; the minimising k at every i is
  the offline policy.

Readings (also in the design notes): q[m] is the draft probability of
reference token m + 1 given the prefix up to m, so at position i,
p_j = q[i + j]; a window reaching past the sequence reads p = 0 there (no
token is left to accept, and every such outcome lands on N anyway); equal
expected costs give the shorter draft; the products of Eq. (7) are taken
with j ascending and the sum of Eq. (8) with a ascending, in float64.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def accept_probs(q: Sequence[float], i: int, k: int) -> List[float]:
    """Eq. (7): P(a | k) for a = 0..k at position i."""
    N = len(q)
    p = [float(q[i + j]) if i + j < N else 0.0 for j in range(k)]
    out = []
    pre = 1.0
    for a in range(k):
        out.append(pre * (1.0 - p[a]))
        pre = pre * p[a]
    out.append(pre)
    return out


def expected_cost(q, cost, dp, i: int, k: int) -> float:
    """The bracket of Eq. (8) for one draft length k at position i."""
    N = len(q)
    P = accept_probs(q, i, k)
    acc = 0.0
    for a in range(k + 1):
        acc = acc + P[a] * (float(cost[i][k - 1][a]) + dp[min(i + a + 1, N)])
    return acc


def bellman_policy(q: Sequence[float], cost: np.ndarray, L: int) -> Tuple[np.ndarray, np.ndarray]:
    """Eq. (8) by backward induction: dp [N+1] float64 and the policy k*[N] int32."""
    N = len(q)
    dp = [0.0] * (N + 1)
    policy = np.zeros(N, dtype=np.int32)
    for i in range(N - 1, -1, -1):
        best, kb = None, 0
        for k in range(1, L + 1):
            v = expected_cost(q, cost, dp, i, k)
            if best is None or v < best:   # equal costs keep the shorter draft
                best, kb = v, k
        dp[i] = best
        policy[i] = kb
    return np.array(dp, dtype=np.float64), policy
