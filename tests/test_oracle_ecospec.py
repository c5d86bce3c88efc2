"""Pins of the EcoSpec selection oracle ("Less Experts, Faster Decoding",
Sec. 4.2, Algorithm 1, Figure 3).

* Figure 3's worked example (tests/golden/ecospec_fig3.json, with the stated
  numbers and the reading of what the caption leaves out): step 1 selects the
  root t0; at step 2, t1 (higher probability 0.53, three new experts) scores
  0.17 and t2 (two new experts) 0.20, so the final set is {t0, t2}.
* With empty footprints every cost is 0 and the rule ranks by probability
  alone: the selection is the top-gamma nodes by cumulative probability, the
  same set as EVICT's truncated tree T_gamma (Sec. 3.2.1 of the adaptive
  verification page) - a special case that reduces to another routine.
* Prefix consistency (Sec. 4.2): every selection prefix is ancestor-closed.
* The final buffer is the initial buffer united with the selected footprints.
"""
import json
import os
import random

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ecospec_fig3.json")


def fig3():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_figure3_worked_example():
    g = fig3()
    rd, st = g["reading"], g["stated"]
    pred = [set((0, e) for e in es) for es in rd["pred_experts"]]
    r = oracle.ecospec_select(rd["parent"], rd["q"], pred, st["gamma"], rd["eps"])
    names = ["t%d" % t for t in r["selected"]]
    assert names[0] == st["step1_selected"]
    assert names == st["final_selected"]
    step2 = r["steps"][1]
    assert round(step2[1], 2) == st["t1_score"]
    assert round(step2[2], 2) == st["t2_score"]
    assert r["P"][1] == pytest.approx(st["t1_cumulative_probability"])
    assert r["P"][1] > r["P"][2]  # the higher-probability candidate loses on cost
    B = r["buffer"]
    assert B == set((0, e) for e in (1, 2, 3, 4, 5, 6))


def random_tree(rng, n):
    return [-1 if v == 0 or rng.random() < 0.15 else rng.randrange(v) for v in range(n)]


def random_probs(rng, n, p_one=0.0):
    return [1.0 if rng.random() < p_one else rng.uniform(0.05, 0.95) for _ in range(n)]


@pytest.mark.parametrize("seed", range(8))
def test_empty_footprints_reduce_to_top_probability(seed):
    rng = random.Random(seed)
    n = rng.randint(1, 30)
    parent, q = random_tree(rng, n), random_probs(rng, n, p_one=0.2)
    gamma = rng.randint(1, n)
    r = oracle.ecospec_select(parent, q, [set() for _ in range(n)], gamma, eps=0.5)
    ev = oracle.evict_select(parent, q, [1.0] * n)
    assert r["selected"] == ev["order"][:gamma]


@pytest.mark.parametrize("seed", range(12))
def test_every_prefix_is_ancestor_closed(seed):
    rng = random.Random(50 + seed)
    n = rng.randint(2, 40)
    parent, q = random_tree(rng, n), random_probs(rng, n, p_one=0.25 if seed % 2 else 0.0)
    L, E = 3, 16
    pred = [set((rng.randrange(L), rng.randrange(E)) for _ in range(rng.randint(0, 5)))
            for _ in range(n)]
    r = oracle.ecospec_select(parent, q, pred, n, eps=rng.choice([1e-3, 0.1, 1.0]))
    for k in range(1, n + 1):
        assert oracle.is_ancestor_closed(parent, r["selected"][:k]), (k, r["selected"])
    traj = oracle.path_footprints(parent, pred)
    assert r["buffer"] == set().union(*[traj[t] for t in r["selected"]])


def test_initial_buffer_makes_covered_experts_free():
    parent = [-1, -1]
    q = [0.5, 0.4]
    pred = [{(0, 1), (0, 2)}, {(0, 3)}]
    # without a buffer: 0.4/1.1 = 0.364 beats 0.5/2.1 = 0.238
    assert oracle.ecospec_select(parent, q, pred, 1, 0.1)["selected"] == [1]
    # with t0's experts already buffered, t0 costs nothing and wins
    assert oracle.ecospec_select(parent, q, pred, 1, 0.1, buffer0={(0, 1), (0, 2)})["selected"] == [0]


def test_bitset_layout_of_the_input_generator():
    from synth.gen import expert_bitsets
    # bit l*experts + e: (1, 3) -> 43 in word 0, (1, 30) -> 70 = word 1, bit 6
    bits = expert_bitsets([{(0, 0), (1, 3), (1, 30)}, set()], layers=2, experts=40)
    assert bits.shape == (2, 2)
    assert int(bits[0, 0]) == 1 | (1 << 43) and int(bits[0, 1]) == 1 << 6
    assert not bits[1].any()
