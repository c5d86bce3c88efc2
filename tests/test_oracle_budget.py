"""Pins of the oracle's per-layer expert budget (MoE-Spec page, abstract).

Against: brute force over every C-subset of the union (the kept set holds the
largest total contribution), contributions recounted with numpy's weighted
bincount (a library formulation the oracle's loop does not use), hand-worked
examples of the grouping arrays and of the tie rule, the identity when the
budget is not binding, and the closed form at one token: a budget of C with
renormalised gates is routing with C experts per token (the softmax over the
top-K logits restricted to its first C entries and renormalised is the
softmax over the top C).
"""
import dataclasses
import itertools

import numpy as np
import pytest

import oracle
from oracle.budget_ref import apply_budget, expert_scores, kept_experts, verify_op_budget
from synth import make_case
from synth.configs import DSV2LITE, TINY


def _random_routing(g, n, K, E):
    ids = np.stack([g.choice(E, size=K, replace=False) for _ in range(n)]).astype(np.int32)
    raw = g.random((n, K))
    gates = raw / raw.sum(axis=1, keepdims=True)
    return ids, gates


def test_hand_example_arrays():
    ids = np.array([[0, 1], [0, 2]], dtype=np.int32)
    gates = np.array([[0.7, 0.3], [0.6, 0.4]])
    un = oracle.build_union(ids, 3)
    b = apply_budget(ids, gates, un, 2)
    # contributions: expert 0 -> 1.3, expert 1 -> 0.3, expert 2 -> 0.4
    assert b["kept"] == [0, 2]
    assert b["U"] == 2
    assert b["union_ids"].tolist() == [0, 2, -1]
    assert b["offsets"].tolist() == [0, 2, 3, 3]
    assert b["perm"].tolist() == [0, 2, 3, 1]
    assert b["slot_rank"].tolist() == [0, -1, 0, 1]
    assert np.array_equal(b["gates"], np.array([[0.7, 0.0], [0.6, 0.4]]))
    r = apply_budget(ids, gates, un, 2, renorm=True)
    assert np.allclose(r["gates"], np.array([[1.0, 0.0], [0.6, 0.4]]), rtol=0, atol=1e-15)


def test_equal_contributions_keep_lower_ids():
    ids = np.array([[3, 1], [2, 0]], dtype=np.int32)
    gates = np.full((2, 2), 0.5)
    un = oracle.build_union(ids, 4)
    assert apply_budget(ids, gates, un, 2)["kept"] == [0, 1]
    assert apply_budget(ids, gates, un, 3)["kept"] == [0, 1, 2]


def test_nan_contribution_ranks_last():
    un = {"U": 3, "union_ids": np.array([0, 1, 2], dtype=np.int32)}
    scores = np.array([np.nan, 0.1, 0.2], dtype=np.float32)
    assert kept_experts(un, scores, 2) == [1, 2]
    assert kept_experts(un, scores, 3) == [0, 1, 2]
    zeros = np.array([-0.0, 0.0, 0.0], dtype=np.float32)
    assert kept_experts(un, zeros, 1) == [0]   # -0.0 equals +0.0: the lower id


@pytest.mark.parametrize("seed", range(6))
def test_contributions_match_weighted_bincount(seed):
    g = np.random.default_rng(100 + seed)
    n, K, E = 5, 3, 9
    ids, gates = _random_routing(g, n, K, E)
    un = oracle.build_union(ids, E)
    sc = expert_scores(un, gates)
    ref = np.bincount(ids.reshape(-1), weights=gates.reshape(-1), minlength=E)
    for u in range(un["U"]):
        assert abs(float(sc[u]) - ref[un["union_ids"][u]]) <= 1e-14


@pytest.mark.parametrize("seed", range(8))
def test_kept_set_is_best_subset_brute_force(seed):
    g = np.random.default_rng(200 + seed)
    n, K, E = 4, 3, 10
    ids, gates = _random_routing(g, n, K, E)
    un = oracle.build_union(ids, E)
    U = un["U"]
    ref = np.bincount(ids.reshape(-1), weights=gates.reshape(-1), minlength=E)
    for C in range(1, U + 1):
        kept = apply_budget(ids, gates, un, C)["kept"]
        best = max(sum(ref[e] for e in sub)
                   for sub in itertools.combinations(un["union_ids"][:U].tolist(), C))
        assert len(kept) == C
        assert abs(sum(ref[e] for e in kept) - best) <= 1e-6


@pytest.mark.parametrize("seed", range(4))
def test_structure_of_budgeted_union(seed):
    g = np.random.default_rng(300 + seed)
    n, K, E = 6, 4, 16
    ids, gates = _random_routing(g, n, K, E)
    un = oracle.build_union(ids, E)
    flat = ids.reshape(-1)
    for C in range(1, un["U"] + 2):
        b = apply_budget(ids, gates, un, C)
        Uk = b["U"]
        assert Uk == min(C, un["U"])
        assert sorted(b["perm"].tolist()) == list(range(n * K))
        off = b["offsets"]
        assert off[0] == 0 and all(off[i] <= off[i + 1] for i in range(len(off) - 1))
        keep = set(b["kept"])
        nkept = sum(1 for s in flat if s in keep)
        assert off[Uk] == nkept and all(v == nkept for v in off[Uk:])
        for u in range(Uk):
            grp = b["perm"][off[u]:off[u + 1]].tolist()
            assert grp == sorted(grp)
            assert all(flat[s] == b["union_ids"][u] for s in grp)
        dropped = b["perm"][nkept:].tolist()
        assert dropped == sorted(dropped) and all(flat[s] not in keep for s in dropped)
        for s in range(n * K):
            r = b["slot_rank"][s]
            assert (r == -1) == (flat[s] not in keep)
            if r >= 0:
                assert b["union_ids"][r] == flat[s]
        assert np.all(b["gates"][~np.isin(ids, list(keep))] == 0.0)


@pytest.mark.parametrize("renorm", [False, True])
def test_budget_not_binding_is_identity(renorm):
    case = make_case(TINY, 4, seed=0)
    plain = oracle.verify_op(case, "dedup")
    U = plain["union"]["U"]
    for C in (U, U + 3):
        b = verify_op_budget(case, C, renorm=renorm)
        assert np.array_equal(b["out"], plain["out"])
        for key in ("union_ids", "offsets", "perm", "slot_rank"):
            assert np.array_equal(b["union"][key], plain["union"][key])
        assert b["union_bytes"] == plain["union_bytes"]


@pytest.mark.parametrize("C", [1, 2, 3])
def test_one_token_budget_equals_routing_with_C_experts(C):
    cfg = dataclasses.replace(TINY, K=4)
    case = make_case(cfg, 1, seed=1)
    b = verify_op_budget(case, C, renorm=True)
    ids_c, gates_c = oracle.route_topk(case.logits, C)
    y, _, _ = oracle.ffn_perslot(case.x, ids_c, case.expert, case.shared, 0, cfg.w_dtype,
                                 cfg.x_dtype, cfg.d, cfg.f)
    ref = oracle.combine(y, gates_c, None)
    assert np.allclose(b["out"], ref, rtol=1e-12, atol=1e-12)
    assert b["union"]["kept"] == sorted(ids_c[0].tolist())


@pytest.mark.parametrize("renorm", [False, True])
def test_dropped_slots_contribute_nothing(renorm):
    cfg = dataclasses.replace(DSV2LITE, d=256, f=128)
    case = make_case(cfg, 3, seed=2)
    ids, gates = oracle.route_topk(case.logits, cfg.K)
    y, ysh, _ = oracle.ffn_perslot(case.x, ids, case.expert, case.shared, cfg.S, cfg.w_dtype,
                                   cfg.x_dtype, cfg.d, cfg.f)
    U = oracle.union_size(ids)
    C = max(1, U - 4)
    b = verify_op_budget(case, C, renorm=renorm)
    keep = np.isin(ids, b["union"]["kept"])
    g = np.where(keep, gates, 0.0)
    if renorm:
        tot = g.sum(axis=1, keepdims=True)
        lost = (~keep).any(axis=1, keepdims=True)
        g = np.where(lost, np.divide(g, tot, out=np.zeros_like(g), where=tot > 0), g)
    ref = np.einsum("tk,tkd->td", g, y) + ysh.sum(axis=1)
    assert np.allclose(b["out"], ref, rtol=1e-12, atol=1e-12)
    assert np.all(b["y_slots"][~keep] == 0.0)
    eb = oracle.expert_bytes(cfg.d, cfg.f, cfg.w_dtype)
    assert b["union_bytes"] == (min(U, C) + cfg.S) * eb
    assert b["requested_bytes"] == 3 * (cfg.K + cfg.S) * eb
