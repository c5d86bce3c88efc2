"""Measurement model of the expert operation (host-side arithmetic on timings).

From "Speculative Decoding for Mixture-of-Experts Models: Expert Bytes,
Kernel Bandwidth and the Best Draft Length":

* a step's time is the bytes each kernel requests over its effective
  bandwidth, plus fixed time (abstract);
* the per-slot kernel's bandwidth is taken on requested bytes n*m*b, the
  deduplicating kernel's on union bytes U*b (Fig. 2);
* u(n) (union share of per-slot bytes) and r(n) = beta_dedup / beta_slot are
  ratios of sums over layers and windows (Table 1 caption);
* deduplication is faster exactly where u(n) < r(n) (Eq. (7));
* the predicted and measured faster kernel agree when
  |ln r - ln u| > ln((1 + eps) / (1 - eps)) for a relative bandwidth error
  eps (Table 2, Eq. (19));
* the crossover is the first pass size at which deduplication is faster
  (abstract; Table 3).

The per-slot re-read model (the page's Eq. (4) is not printed; reading):
tau_slot = t0 + b * (c_u * U + c_re * (n*m - U)), a first read of an
expert costs c_u per byte and every repeat c_re.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


def ratio_of_sums(num: Iterable[float], den: Iterable[float]) -> float:
    num, den = list(num), list(den)
    return float(sum(num)) / float(sum(den))


def aggregate(ops: Sequence[Dict[str, float]]) -> Dict[str, float]:
    """ops: dicts with union_bytes, requested_bytes, t_dedup, t_slot (seconds)."""
    u = ratio_of_sums((o["union_bytes"] for o in ops), (o["requested_bytes"] for o in ops))
    beta_d = ratio_of_sums((o["union_bytes"] for o in ops), (o["t_dedup"] for o in ops))
    beta_s = ratio_of_sums((o["requested_bytes"] for o in ops), (o["t_slot"] for o in ops))
    saving = float(np.mean([o["t_slot"] - o["t_dedup"] for o in ops]))
    return {"u": u, "beta_dedup": beta_d, "beta_slot": beta_s, "r": beta_d / beta_s,
            "saving": saving}


def dedup_faster(u: float, r: float) -> bool:
    """Eq. (7): deduplication wins where its byte share is below its bandwidth ratio."""
    return u < r


def sign_is_robust(r: float, u: float, eps: float) -> bool:
    """Eq. (19): the sides of Eq. (7) keep their order under a relative bandwidth error eps."""
    return abs(math.log(r) - math.log(u)) > math.log((1 + eps) / (1 - eps))


def crossover(ns: Sequence[int], savings: Sequence[float]) -> Optional[int]:
    for n, s in zip(ns, savings):
        if s > 0:
            return n
    return None


def fit_bandwidth(bytes_: Sequence[float], times: Sequence[float]) -> Tuple[float, float]:
    """Least squares of tau = bytes / beta + t0; returns (beta, t0)."""
    a = np.vstack([np.asarray(bytes_, dtype=np.float64), np.ones(len(bytes_))]).T
    slope, t0 = np.linalg.lstsq(a, np.asarray(times, dtype=np.float64), rcond=None)[0]
    return (1.0 / slope if slope > 0 else float("inf")), float(t0)


def fit_reread(U: Sequence[int], nm: Sequence[int], b: float,
               t_slot: Sequence[float]) -> Dict[str, float]:
    """tau_slot = t0 + b (c_u U + c_re (n m - U)); returns c_u, c_re (s/byte), t0 and c_re/c_u."""
    U = np.asarray(U, dtype=np.float64)
    rep = np.asarray(nm, dtype=np.float64) - U
    a = np.vstack([b * U, b * rep, np.ones(len(U))]).T
    c_u, c_re, t0 = np.linalg.lstsq(a, np.asarray(t_slot, dtype=np.float64), rcond=None)[0]
    return {"c_u": float(c_u), "c_re": float(c_re), "t0": float(t0),
            "reread_cost": float(c_re / c_u) if c_u != 0 else float("nan")}


# ------------------------------------------------------------------------
# Best draft length under geometric acceptance (expert-bytes page: abstract;
# appendix symbol table: a, a_0 = V(1)/V(0) - 1, step points a_j,
# c_i = V(i) - V(i-1); Table 2, Eqs. (17), (18), (20), (21)).
#
# Reading (the page's body is not printed): a step with k drafted tokens
# verifies k + 1 positions and takes V(k) = tau(k + 1); each draft is accepted
# with probability a, independently, until the first rejection, and the step
# commits the accepted drafts plus one token of the target, so it commits
# sum_{j=0..k} a^j tokens on average.  Throughput T_a(k) = that sum / V(k);
# the best draft length k*(a) maximises it (ties: the shorter draft).


def expected_tokens(k: int, a: float) -> float:
    """Tokens one step with k drafts commits on average: sum_{j=0..k} a^j."""
    return float(sum(a ** j for j in range(k + 1)))


def throughput(V: Sequence[float], a: float) -> List[float]:
    """T_a(k) = sum_{j<=k} a^j / V(k) for k = 0 .. len(V) - 1 (tokens per unit of V)."""
    return [expected_tokens(k, a) / float(v) for k, v in enumerate(V)]


def best_draft_length(V: Sequence[float], a: float) -> int:
    """k*(a) = argmax_k T_a(k); on equal throughput the shorter draft."""
    t = throughput(V, a)
    best = 0
    for k in range(1, len(t)):
        if t[k] > t[best]:
            best = k
    return best


def a0(V: Sequence[float]) -> float:
    """The acceptance above which one draft is faster than none: V(1)/V(0) - 1."""
    return float(V[1]) / float(V[0]) - 1.0


def step_points(V: Sequence[float], tol: float = 1e-12) -> List[Tuple[float, int]]:
    """The staircase k*(a) on [0, 1): [(a_j, k after the step)], found by
    bisection between the acceptance values where k* changes (k* is
    nondecreasing in a, the page's staircase)."""
    out: List[Tuple[float, int]] = []
    lo_k = best_draft_length(V, 0.0)
    a_lo = 0.0
    top = 1.0 - 1e-9
    while True:
        k_top = best_draft_length(V, top)
        if k_top == lo_k:
            return out
        lo, hi = a_lo, top  # k*(lo) == lo_k, k*(hi) > lo_k
        while hi - lo > tol:
            mid = 0.5 * (lo + hi)
            if best_draft_length(V, mid) == lo_k:
                lo = mid
            else:
                hi = mid
        new_k = best_draft_length(V, hi)
        out.append((hi, new_k))
        lo_k, a_lo = new_k, hi


def step_costs(V: Sequence[float]) -> List[float]:
    """c_i = V(i) - V(i-1), the time the i-th draft adds (i >= 1)."""
    return [float(V[i]) - float(V[i - 1]) for i in range(1, len(V))]


# --- Table 2: error bounds -------------------------------------------------

def verify_time_bound(M: float, eps: float) -> float:
    """Eq. (17): |tau_hat - tau| <= eps/(1-eps) M for a relative bandwidth error
    eps, M = the bytes-over-bandwidth part of tau."""
    return eps / (1.0 - eps) * M


def saving_bound(M_slot: float, M_dedup: float, eps: float) -> float:
    """Eq. (18): |S_hat - S| <= eps/(1-eps) (M_slot + M_dedup)."""
    return eps / (1.0 - eps) * (M_slot + M_dedup)


def draft_length_loss_bound(delta: float) -> float:
    """Eq. (20): with step times known to a relative error delta, the predicted
    best draft length loses at most 2 delta / (1 + delta) of the throughput."""
    return 2.0 * delta / (1.0 + delta)


def best_draft_length_certain(V: Sequence[float], a: float, delta: float) -> bool:
    """Eq. (20): the predicted k* is the true one when
    (1+delta)/(1-delta) T_a(i) < T_a(k*) for every i != k*."""
    t = throughput(V, a)
    k = best_draft_length(V, a)
    f = (1.0 + delta) / (1.0 - delta)
    return all(f * t[i] < t[k] for i in range(len(t)) if i != k)


def speedup_interval(delta: float) -> Tuple[float, float]:
    """Eq. (21): predicted best speedup over true best speedup lies in
    [(1-delta)/(1+delta), (1+delta)/(1-delta)]."""
    return (1.0 - delta) / (1.0 + delta), (1.0 + delta) / (1.0 - delta)


# --- "The Limits of Speculation" page, Sec. 3 -----------------------------

def eta(V: Sequence[float]) -> List[float]:
    """Eq. (1): target efficiency eta(K) = T_T(0) / T_T(K) (here T_T(K) = V(K))."""
    return [float(V[0]) / float(v) for v in V]


def speedup_limits(mean_gain: float, K: int, t_draft: float, t_target0: float,
                   eta_k: float) -> float:
    """Eq. (2): SpeedUp ~ E[G] / (K T_D / T_T(0) + 1 / eta(K))."""
    return mean_gain / (K * t_draft / t_target0 + 1.0 / eta_k)
