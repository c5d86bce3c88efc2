"""Routing statistics: exact brute force against the closed forms, and the generators.

Under independent uniform routing of n tokens, each picking K of E experts,
the expected union is E (1 - q^n) with q = 1 - K/E, and the expected share of
the last token's experts already chosen by the n - 1 before it is
1 - q^(n-1) (expert-bytes page, Figure 1: the dotted independent-routing
curve of consecutive-token reuse).  The enumeration below visits every
routing of tiny (E, K, n) and sums with exact rationals; the oracle supplies
only the per-routing union size and reuse.

The Markov generator keeps each of the predecessor's experts with
probability p, so the overlap with the predecessor is Binomial(K, p) and
E[U(n=2)] = K (2 - p).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth.configs import DSV3, OLMOE, QWEN3
from synth.gen import chain_parents, iid_sets, markov_sets, tree_parents


def _exact_expectations(E, K, n):
    sets = list(itertools.combinations(range(E), K))
    total_u = Fraction(0)
    total_r = Fraction(0)
    count = 0
    for routing in itertools.product(sets, repeat=n):
        ids = np.array(routing, dtype=np.int32)
        total_u += oracle.union_size(ids)
        total_r += Fraction(oracle.reuse_last(ids)).limit_denominator(K)
        count += 1
    return total_u / count, total_r / count


@pytest.mark.parametrize("E,K,n,eu,rho", [
    (4, 1, 3, Fraction(37, 16), Fraction(7, 16)),
    (5, 2, 2, Fraction(16, 5), Fraction(2, 5)),
    (6, 2, 3, Fraction(38, 9), Fraction(5, 9)),
    (8, 2, 4, Fraction(175, 32), Fraction(37, 64)),
])
def test_exact_union_and_reuse_match_closed_forms(E, K, n, eu, rho):
    mean_u, mean_r = _exact_expectations(E, K, n)
    q = 1 - Fraction(K, E)
    assert mean_u == E * (1 - q ** n) == eu
    assert mean_r == 1 - q ** (n - 1) == rho


@pytest.mark.parametrize("cfg,n", [(OLMOE, 2), (OLMOE, 8), (QWEN3, 4), (DSV3, 8), (DSV3, 32)])
def test_monte_carlo_union_at_layer_sizes(cfg, n):
    g = np.random.default_rng(100 + n)
    trials = 1500
    us = np.array([oracle.union_size(iid_sets(g, n, cfg.E, cfg.K)) for _ in range(trials)])
    q = 1 - cfg.K / cfg.E
    expect = cfg.E * (1 - q ** n)
    assert abs(us.mean() - expect) < 3.5 * us.std(ddof=1) / np.sqrt(trials) + 1e-9


@pytest.mark.parametrize("p", [0.0, 0.5, 0.8, 1.0])
def test_markov_overlap_is_binomial_and_two_token_union(p):
    g = np.random.default_rng(int(p * 10))
    E, K = OLMOE.E, OLMOE.K
    trials = 3000
    overlaps = []
    unions = []
    for _ in range(trials):
        ids = markov_sets(g, chain_parents(2), E, K, p)
        assert len(set(ids[1].tolist())) == K           # K distinct per token
        overlaps.append(len(set(ids[0].tolist()) & set(ids[1].tolist())))
        unions.append(oracle.union_size(ids))
    overlaps = np.array(overlaps, dtype=np.float64)
    unions = np.array(unions, dtype=np.float64)
    if p in (0.0, 1.0):
        assert np.all(overlaps == K * p)
        assert np.all(unions == K * (2 - p))
        return
    se = np.sqrt(K * p * (1 - p) / trials)
    assert abs(overlaps.mean() - K * p) < 4 * se
    assert abs(overlaps.var(ddof=1) - K * p * (1 - p)) < 0.15 * K * p * (1 - p)
    assert abs(unions.mean() - K * (2 - p)) < 4 * se


def test_tree_parents_heap_shape():
    p = tree_parents(7)
    assert p.tolist() == [-1, 0, 0, 1, 1, 2, 2]


def test_distinct_share_bounds():
    g = np.random.default_rng(4)
    for n in (1, 2, 4, 8):
        for _ in range(50):
            ids = markov_sets(g, chain_parents(n), 64, 8, 0.5)
            share = oracle.distinct_share(ids)
            assert 1.0 / n <= share <= 1.0
