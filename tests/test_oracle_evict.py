"""Pins of the EVICT truncation oracle ("Making Every Verified Token Count",
Sec. 2.1, Sec. 3.1-3.2, App. A).

* App. A: the expected accepted length of a tree equals the sum over nodes of
  the path products of the target probabilities (Eq. (6)/(14)).  Pinned by
  enumerating every outcome of the sequential verification rule of Sec. 2.1
  (children tried in turn, accepted with their probability, rejected mass
  removed and the rest renormalised, Eq. (3)) on small trees: the oracle's
  score sum with q = p must equal that expectation exactly (Fractions).
* Sec. 3.2.1: every T_k is ancestor-closed, and its score sum is the largest
  over all ancestor-closed k-node subtrees (brute force over all subsets).
* Eq. (10): k* equals a brute-force argmax over k of E_hat(T_k) / C(k).
"""
import itertools
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle


def random_tree(rng, n, max_children=3):
    parent = []
    for v in range(n):
        cands = [-1] + [u for u in range(v) if sum(1 for p in parent if p == u) < max_children]
        parent.append(rng.choice(cands))
    return parent


def sibling_probs(rng, parent, exact=False):
    """Draft/target conditional probabilities of every node: the children of
    one node share at most probability 1."""
    q = [0.0] * len(parent)
    groups = {}
    for v, p in enumerate(parent):
        groups.setdefault(p, []).append(v)
    for p, kids in groups.items():
        w = [rng.randint(1, 9) for _ in range(len(kids) + 1)]  # the last share: no child
        tot = sum(w)
        for v, wi in zip(kids, w):
            q[v] = Fraction(wi, tot) if exact else wi / tot
    return q


def accepted_length_by_rule(parent, p):
    """Exact E[accepted length] under the sequential rule of Sec. 2.1."""
    kids = {}
    for v, u in enumerate(parent):
        kids.setdefault(u, []).append(v)

    def expect(u):
        # expected number of further accepted nodes below u (u already accepted)
        ch = kids.get(u, [])
        total = Fraction(0)
        remaining = Fraction(1)   # probability that all earlier siblings were rejected
        dist = {c: p[c] for c in ch}
        for c in ch:
            mass = dist[c]
            # accept c with its current (renormalised) probability
            total += remaining * mass * (1 + expect(c))
            remaining *= (1 - mass)
            # Eq. (3): remove c's mass, renormalise the rest
            if 1 - mass != 0:
                for w in ch:
                    if w != c:
                        dist[w] = dist[w] / (1 - mass)
            dist[c] = Fraction(0)
        return total

    return expect(-1)


@pytest.mark.parametrize("seed", range(12))
def test_score_sum_is_expected_accepted_length(seed):
    rng = random.Random(seed)
    parent = random_tree(rng, rng.randint(1, 7))
    p = sibling_probs(rng, parent, exact=True)
    ref = accepted_length_by_rule(parent, p)
    # the oracle's scores with q = p (products in float64; the Fractions are
    # exact, so compare to rounding)
    s = oracle.path_scores(parent, [float(x) for x in p])
    assert float(ref) == pytest.approx(float(np.sum(s)), rel=1e-6)


def test_rule_enumeration_on_a_chain_and_a_star():
    # chain: E = p1 + p1 p2 + p1 p2 p3; star: E = sum of the children's p
    chain = [-1, 0, 1]
    pc = [Fraction(1, 2), Fraction(1, 3), Fraction(1, 4)]
    assert accepted_length_by_rule(chain, pc) == Fraction(1, 2) + Fraction(1, 6) + Fraction(1, 24)
    star = [-1, -1, -1]
    ps = [Fraction(1, 5), Fraction(2, 5), Fraction(1, 5)]
    assert accepted_length_by_rule(star, ps) == Fraction(4, 5)


@pytest.mark.parametrize("seed", range(10))
def test_topk_is_ancestor_closed_and_optimal(seed):
    rng = random.Random(100 + seed)
    n = rng.randint(1, 8)
    parent = random_tree(rng, n)
    q = sibling_probs(rng, parent)
    if seed % 3 == 0:  # some probability-1 edges: equal scores of parent and child
        for v in range(n):
            if rng.random() < 0.3:
                q[v] = 1.0
    r = oracle.evict_select(parent, q, [1.0] * n)
    s = r["scores"]
    for k in range(1, n + 1):
        top = r["order"][:k]
        assert oracle.is_ancestor_closed(parent, top)
        best = max(sum(s[v] for v in sub) for sub in itertools.combinations(range(n), k)
                   if oracle.is_ancestor_closed(parent, sub))
        assert r["expected"][k - 1] == pytest.approx(best, rel=1e-12)


@pytest.mark.parametrize("seed", range(10))
def test_k_best_is_the_utility_argmax(seed):
    rng = random.Random(200 + seed)
    n = rng.randint(1, 40)
    parent = random_tree(rng, n)
    q = sibling_probs(rng, parent)
    cost = sorted(rng.uniform(1.0, 3.0) for _ in range(n))
    r = oracle.evict_select(parent, q, cost)
    s = r["scores"]
    util = []
    for k in range(1, n + 1):
        chosen = sorted(range(n), key=lambda v: (-s[v], v))[:k]
        util.append(sum(s[v] for v in chosen) / float(np.float32(cost[k - 1])))
    assert r["k_best"] == 1 + max(range(n), key=lambda i: (util[i], -i))


def test_constant_cost_keeps_everything_and_steep_cost_keeps_one():
    parent = [-1, 0, 0, 1]
    q = [0.9, 0.5, 0.4, 0.8]
    assert oracle.evict_select(parent, q, [1.0] * 4)["k_best"] == 4
    assert oracle.evict_select(parent, q, [1.0, 10.0, 20.0, 40.0])["k_best"] == 1
