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
