"""Pins of the oracle's router top-K and expert union.

Top-K (adaptive-verification page, Sec. 2.2, Eq. (4)): the K largest router
scores, normalised over the K.  Union (cost-aware page, Sec. 3, Eq. (1);
adaptive-verification page, Eq. (5); limits page, App. A.4.1, Eq. (A2)):
the distinct experts over all verified tokens.  Bounds on U / (n m) are from
the expert-bytes page, Figure 3 (right): between 1/n and 1.

The references are independent: a selection-by-repeated-scan for top-K, a
counting sort for the permutation, Python sets for the union, and closed
forms for the softmax of two values.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle


# ------------------------------------------------------------------- top-K
def _scan_topk(row, K):
    """Repeatedly take the best remaining expert: largest number, NaN last, lower id on ties."""
    taken = []
    for _ in range(K):
        best = None
        for e, v in enumerate(row):
            if e in taken:
                continue
            if best is None:
                best = e
                continue
            b = row[best]
            if math.isnan(b) and not math.isnan(v):
                best = e
            elif not math.isnan(b) and not math.isnan(v) and v > b:
                best = e
        taken.append(best)
    return taken


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 4), st.integers(1, 12), st.data())
def test_topk_matches_repeated_scan(n, E, data):
    K = data.draw(st.integers(1, E))
    # small integer-valued logits force many ties; some NaNs and signed zeros
    vals = data.draw(st.lists(st.sampled_from([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, float("nan")]),
                              min_size=n * E, max_size=n * E))
    logits = np.array(vals, dtype=np.float32).reshape(n, E)
    ids, gates = oracle.route_topk(logits, K)
    for t in range(n):
        assert list(ids[t]) == _scan_topk([float(v) for v in logits[t]], K)


def test_topk_all_experts_when_K_equals_E():
    lg = np.array([[0.3, -1.0, 2.0, 0.3]], dtype=np.float32)
    ids, gates = oracle.route_topk(lg, 4)
    assert list(ids[0]) == [2, 0, 3, 1]
    assert abs(gates.sum() - 1.0) < 1e-15


def test_topk_equal_logits_take_lowest_ids():
    ids, gates = oracle.route_topk(np.zeros((2, 9), dtype=np.float32), 3)
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    assert np.allclose(gates, 1.0 / 3.0, rtol=0, atol=1e-15)


def test_topk_signed_zeros_tie():
    lg = np.array([[-0.0, 0.0, -5.0]], dtype=np.float32)
    ids, _ = oracle.route_topk(lg, 1)
    assert ids[0, 0] == 0


def test_topk_nan_never_beats_a_number():
    lg = np.array([[float("nan"), -1e30, float("nan"), -3.0]], dtype=np.float32)
    ids, _ = oracle.route_topk(lg, 3)
    assert ids[0].tolist() == [3, 1, 0]


@pytest.mark.parametrize("l0,l1", [(1.0, 0.0), (3.5, -2.0), (0.25, 0.25), (10.0, 9.0)])
def test_softmax_of_two_is_a_sigmoid(l0, l1):
    ids, gates = oracle.route_topk(np.array([[l1, l0, -50.0]], dtype=np.float32), 2)
    hi, lo = max(l0, l1), min(l0, l1)
    assert gates[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(lo - hi)), rel=1e-14)
    assert gates[0, 1] == pytest.approx(1.0 / (1.0 + math.exp(hi - lo)), rel=1e-14)


def test_top1_gate_is_one():
    lg = np.random.default_rng(3).standard_normal((5, 16)).astype(np.float32)
    ids, gates = oracle.route_topk(lg, 1)
    assert np.all(gates == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))


# ------------------------------------------------------------------- union
def _counting_sort_perm(flat, E):
    buckets = [[] for _ in range(E)]
    for s, e in enumerate(flat):
        buckets[e].append(s)
    return [s for b in buckets for s in b]


def _random_ids(g, n, E, K):
    return np.stack([g.choice(E, K, replace=False) for _ in range(n)]).astype(np.int32)


@pytest.mark.parametrize("n,E,K", [(1, 8, 2), (4, 8, 2), (8, 64, 8), (16, 64, 6), (32, 256, 8),
                                   (3, 5, 5), (32, 8, 8)])
def test_union_against_sets_and_counting_sort(n, E, K):
    g = np.random.default_rng(n * 1000 + E)
    for _ in range(5):
        ids = _random_ids(g, n, E, K)
        flat = ids.reshape(-1).tolist()
        un = oracle.build_union(ids, E)
        U = un["U"]
        cap = min(n * K, E)
        distinct = sorted(set(flat))
        assert U == len(distinct)
        assert K <= U <= cap
        assert 1.0 / n <= U / (n * K) <= 1.0
        assert un["union_ids"][:U].tolist() == distinct
        assert np.all(un["union_ids"][U:] == -1) and len(un["union_ids"]) == cap
        assert un["perm"].tolist() == _counting_sort_perm(flat, E)
        for u, e in enumerate(distinct):
            assert un["offsets"][u + 1] - un["offsets"][u] == flat.count(e)
        assert un["offsets"][0] == 0 and np.all(un["offsets"][U:] == n * K)
        assert len(un["offsets"]) == cap + 1
        for s, e in enumerate(flat):
            assert un["union_ids"][un["slot_rank"][s]] == e


def test_union_equals_K_iff_all_tokens_share_one_set():
    same = np.array([[3, 1, 4]] * 5, dtype=np.int32)
    assert oracle.build_union(same, 10)["U"] == 3
    diff = same.copy()
    diff[4, 0] = 9
    assert oracle.build_union(diff, 10)["U"] == 4


def test_union_equals_nK_iff_disjoint():
    ids = np.arange(12, dtype=np.int32).reshape(4, 3)
    assert oracle.build_union(ids, 12)["U"] == 12
    ids[3, 2] = 0
    assert oracle.build_union(ids, 12)["U"] == 11


def test_union_rejects_out_of_range_ids():
    assert oracle.build_union(np.array([[0, 8]], dtype=np.int32), 8)["U"] == -1
    assert oracle.build_union(np.array([[-1, 2]], dtype=np.int32), 8)["U"] == -1


def test_perm_is_stable_for_repeated_expert():
    ids = np.array([[5, 2], [2, 7], [7, 5]], dtype=np.int32)
    un = oracle.build_union(ids, 8)
    # expert 2: slots 1, 2; expert 5: slots 0, 5; expert 7: slots 3, 4
    assert un["perm"].tolist() == [1, 2, 0, 5, 3, 4]
    assert un["offsets"].tolist() == [0, 2, 4, 6, 6, 6, 6]
