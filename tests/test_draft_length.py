"""Pins of the best-draft-length arithmetic (expert-bytes page: abstract,
appendix symbol table, Table 2 Eqs. (17)-(21); limits page Eqs. (1)-(2)).

The pins do not retype the formulas: expected committed tokens come from an
enumeration of every accept/reject outcome of the geometric rule, the error
bounds are checked by perturbing step times and bandwidths at random within
the stated error, and the staircase against a fine grid of acceptance values.
"""
import itertools
import math
import random
from fractions import Fraction

import pytest

from moe_speculative_decoding_amd import costmodel as cm


def committed_by_enumeration(k, a):
    """Every draft gets an independent accept flag (probability a); the step
    commits the drafts before the first rejected one, plus one token of the
    target.  Exact expectation over all 2^k flag sequences."""
    total = Fraction(0)
    for flags in itertools.product((True, False), repeat=k):
        p = Fraction(1)
        for ok in flags:
            p *= a if ok else (1 - a)
        leading = next((i for i, ok in enumerate(flags) if not ok), k)
        total += p * (leading + 1)
    return total


@pytest.mark.parametrize("k", [0, 1, 2, 3, 5, 8])
@pytest.mark.parametrize("a", [Fraction(0), Fraction(1, 3), Fraction(7, 10), Fraction(1)])
def test_expected_tokens_geometric_rule(k, a):
    ref = committed_by_enumeration(k, a)
    assert cm.expected_tokens(k, float(a)) == pytest.approx(float(ref), rel=1e-12, abs=1e-12)


def test_throughput_closed_form():
    V = [1.0, 1.3, 1.5, 1.9, 2.6]
    for a in (0.0, 0.2, 0.55, 0.9):
        t = cm.throughput(V, a)
        for k, v in enumerate(V):
            assert t[k] == pytest.approx((1 - a ** (k + 1)) / (1 - a) / v, rel=1e-12)


def test_a0_is_where_one_draft_starts_to_pay():
    V = [1.0, 1.25, 1.6, 2.2]
    a = cm.a0(V)
    assert a == pytest.approx(0.25)
    t_lo, t_hi = cm.throughput(V, a - 1e-6), cm.throughput(V, a + 1e-6)
    assert t_lo[1] < t_lo[0] and t_hi[1] > t_hi[0]
    pts = cm.step_points(V)
    assert pts[0][1] == 1 and pts[0][0] == pytest.approx(a, abs=1e-9)


def _random_steps(rng, n):
    # nondecreasing step times with a fixed part: V(k) = t0 + sum of increments
    t0 = rng.uniform(0.2, 2.0)
    inc = [rng.uniform(0.0, 0.5) for _ in range(n - 1)]
    V = [t0]
    for d in inc:
        V.append(V[-1] + d)
    return V


def test_staircase_is_monotone_and_matches_grid():
    rng = random.Random(7)
    for _ in range(40):
        V = _random_steps(rng, rng.randint(2, 9))
        grid = [i / 2000 for i in range(2000)]
        ks = [cm.best_draft_length(V, a) for a in grid]
        assert all(x <= y for x, y in zip(ks, ks[1:])), V
        pts = cm.step_points(V)
        for a, k in zip(grid, ks):
            if any(abs(a - aa) <= 1e-9 for aa, _ in pts):
                continue  # within the bisection tolerance of a step
            before = [kk for (aa, kk) in pts if aa <= a]
            assert k == (before[-1] if before else cm.best_draft_length(V, 0.0))


def test_step_costs_are_increments():
    V = [2.0, 2.5, 3.25]
    assert cm.step_costs(V) == [0.5, 0.75]


def test_eq20_eq21_under_random_step_time_errors():
    rng = random.Random(11)
    for _ in range(300):
        V = _random_steps(rng, rng.randint(2, 9))
        a = rng.uniform(0.0, 0.98)
        delta = rng.uniform(0.0, 0.3)
        V_hat = [v * (1 + rng.uniform(-delta, delta)) for v in V]
        t = cm.throughput(V, a)
        k_true = cm.best_draft_length(V, a)
        k_hat = cm.best_draft_length(V_hat, a)
        assert t[k_hat] >= (1 - delta) / (1 + delta) * t[k_true] - 1e-15
        assert 1 - t[k_hat] / t[k_true] <= cm.draft_length_loss_bound(delta) + 1e-12
        if cm.best_draft_length_certain(V, a, delta):
            assert k_hat == k_true
        th = cm.throughput(V_hat, a)
        lo, hi = cm.speedup_interval(delta)
        ratio = (th[k_hat] / th[0]) / (t[k_true] / t[0])
        assert lo - 1e-12 <= ratio <= hi + 1e-12


def test_eq17_eq18_under_random_bandwidth_errors():
    rng = random.Random(3)
    for _ in range(300):
        eps = rng.uniform(0.0, 0.4)
        t0 = rng.uniform(0.0, 5.0)
        bs, bd = rng.uniform(1e8, 1e9), rng.uniform(1e8, 1e9)
        beta_s, beta_d = rng.uniform(1e11, 8e12), rng.uniform(1e11, 8e12)
        Ms, Md = bs / beta_s, bd / beta_d
        hs = bs / (beta_s * (1 + rng.uniform(-eps, eps)))
        hd = bd / (beta_d * (1 + rng.uniform(-eps, eps)))
        assert abs((hs + t0) - (Ms + t0)) <= cm.verify_time_bound(Ms, eps) * (1 + 1e-12)
        S, S_hat = Ms - Md, hs - hd
        assert abs(S_hat - S) <= cm.saving_bound(Ms, Md, eps) * (1 + 1e-12)


def test_limits_page_eta_and_speedup():
    V = [10.0, 12.0, 15.0, 21.0]
    e = cm.eta(V)
    assert e[0] == 1.0 and all(x > y for x, y in zip(e, e[1:]))
    # no drafts: one committed token per target pass, speedup 1
    assert cm.speedup_limits(1.0, 0, 0.7, V[0], e[0]) == pytest.approx(1.0)
    # free drafts: speedup = E[G] * eta(K)
    assert cm.speedup_limits(2.5, 3, 0.0, V[0], e[3]) == pytest.approx(2.5 * e[3])
