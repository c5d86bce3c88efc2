"""Pins of the oracle's Bellman draft-length oracle ([LS] = "The Limits of
Speculation: Bounding Speculative Decoding in MoE", Sec. 4, Eqs. (7)-(8)).

Against: exact enumeration of every accept/reject flag sequence of a window
(P(a | k) is the probability that the first rejection falls at a), exact
forward enumeration of every outcome path of every deterministic policy on
tiny sequences (the minimum over policies is dp[0], and the oracle's policy
attains it), the telescoping sum of Eq. (7), the mean-acceptance identity,
and the closed forms of always-accepted and never-accepted drafts.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle.bellman_ref import accept_probs, bellman_policy


def _flags_hist(p):
    """P(first rejection at a) by enumerating every flag sequence."""
    k = len(p)
    hist = [Fraction(0)] * (k + 1)
    for flags in itertools.product((0, 1), repeat=k):
        pr = Fraction(1)
        for j, f in enumerate(flags):
            pr *= p[j] if f else (1 - p[j])
        a = flags.index(0) if 0 in flags else k
        hist[a] += pr
    return hist


@pytest.mark.parametrize("seed", range(5))
def test_accept_probs_match_flag_enumeration(seed):
    g = np.random.default_rng(seed)
    N = 7
    qf = [Fraction(int(v), 16) for v in g.integers(0, 17, size=N)]
    q = [float(v) for v in qf]
    for i in range(N):
        for k in range(1, 6):
            p = [qf[i + j] if i + j < N else Fraction(0) for j in range(k)]
            ref = _flags_hist(p)
            got = accept_probs(q, i, k)
            assert len(got) == k + 1
            for a in range(k + 1):
                assert abs(got[a] - float(ref[a])) <= 1e-15


@pytest.mark.parametrize("seed", range(5))
def test_accept_probs_sum_and_mean(seed):
    g = np.random.default_rng(10 + seed)
    q = g.random(20)
    for i in range(0, 20, 3):
        for k in range(1, 9):
            P = accept_probs(q, i, k)
            assert abs(sum(P) - 1.0) <= 1e-14
            mean = sum(a * P[a] for a in range(k + 1))
            p = [q[i + j] if i + j < 20 else 0.0 for j in range(k)]
            ref = sum(math.prod(p[:j]) for j in range(1, k + 1))
            assert abs(mean - ref) <= 1e-14


def _policy_cost(qf, costf, pol, N):
    """Exact expected total cost of a deterministic policy, by enumerating every
    outcome path forward from position 0 (flags drawn token by token)."""
    total = Fraction(0)
    stack = [(0, Fraction(1), Fraction(0))]
    while stack:
        pos, pr, acc = stack.pop()
        if pos >= N:
            total += pr * acc
            continue
        k = pol[pos]
        p = [qf[pos + j] if pos + j < N else Fraction(0) for j in range(k)]
        for a, pa in enumerate(_flags_hist(p)):
            if pa == 0:
                continue
            stack.append((min(pos + a + 1, N), pr * pa, acc + costf[pos][k - 1][a]))
    return total


@pytest.mark.parametrize("N,L,seed", [(3, 2, 0), (4, 2, 1), (4, 3, 2), (5, 2, 3), (3, 3, 4)])
def test_bellman_is_best_policy_by_enumeration(N, L, seed):
    g = np.random.default_rng(100 + seed)
    qf = [Fraction(int(v), 8) for v in g.integers(0, 9, size=N)]
    costf = [[[Fraction(int(g.integers(1, 40)), 4) for _ in range(L + 1)] for _ in range(L)]
             for _ in range(N)]
    q = np.array([float(v) for v in qf])
    cost = np.array([[[float(c) for c in row] for row in blk] for blk in costf])
    dp, pol = bellman_policy(q, cost, L)
    best = min(_policy_cost(qf, costf, pp, N) for pp in itertools.product(range(1, L + 1), repeat=N))
    assert abs(dp[0] - float(best)) <= 1e-12 * max(1.0, float(best))
    assert abs(float(_policy_cost(qf, costf, list(pol), N)) - float(best)) <= 1e-12 * float(best)
    assert dp[N] == 0.0


@pytest.mark.parametrize("N,L", [(10, 3), (17, 4), (6, 8)])
def test_always_accepted_drafts(N, L):
    c = 2.5
    q = np.ones(N)
    cost = np.full((N, L, L + 1), c)
    dp, pol = bellman_policy(q, cost, L)
    for i in range(N):
        assert dp[i] == c * math.ceil((N - i) / (L + 1))
        if N - i <= L + 1:   # one step finishes: the shortest draft that reaches N
            assert pol[i] == max(1, N - i - 1)


def test_never_accepted_drafts_take_the_shortest():
    N, L = 12, 5
    q = np.zeros(N)
    t, T = 0.4, 3.0
    cost = np.array([[[t * k + T] * (L + 1) for k in range(1, L + 1)] for _ in range(N)])
    dp, pol = bellman_policy(q, cost, L)
    assert np.all(pol == 1)
    for i in range(N + 1):
        assert abs(dp[i] - (N - i) * (t + T)) <= 1e-12
