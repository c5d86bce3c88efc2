"""Pins of the measurement model against the expert-bytes page's Table 1 and algebra.

Table 1 prints beta_slot, beta_dedup, r and u for five engine/model pairs at
n = 2 and n = 8; r must equal beta_dedup / beta_slot to the printed two
decimals, and Eq. (7) (dedup faster iff u < r) must reproduce the page's own
statement that the Metal Qwen3 pair has no crossover (Table 3: '-').
"""
import json
import math
import os

import numpy as np
import pytest

from moe_speculative_decoding_amd import costmodel as cm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p4_table1.json")


def rows():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_table1_r_is_bandwidth_ratio():
    # the page prints r to two decimals and each bandwidth to 1 GB/s, both
    # rounded from unrounded sums, so the printed ratio may miss by up to 0.01
    for row in rows()["rows"]:
        assert abs(row["beta_dedup"] / row["beta_slot"] - row["r"]) <= 0.01, row


def test_table1_metal_qwen3_dedup_never_faster():
    t = rows()
    pair = t["crossover_none_at_n8"]
    for row in t["rows"]:
        if row["engine"] == pair["engine"] and row["model"] == pair["model"]:
            assert not cm.dedup_faster(row["u"], row["r"])


def test_mode_criterion_equals_time_comparison():
    # with tau = bytes / beta, tau_dedup < tau_slot  <=>  u < r
    g = np.random.default_rng(0)
    for _ in range(1000):
        req = g.uniform(1e8, 1e9)
        u = g.uniform(0.1, 1.0)
        b_s, b_d = g.uniform(1e11, 8e12, 2)
        t_d, t_s = u * req / b_d, req / b_s
        assert (t_d < t_s) == cm.dedup_faster(u, b_d / b_s)


def test_aggregate_is_ratio_of_sums():
    ops = [dict(union_bytes=10, requested_bytes=20, t_dedup=1.0, t_slot=2.0),
           dict(union_bytes=30, requested_bytes=40, t_dedup=5.0, t_slot=2.0)]
    a = cm.aggregate(ops)
    assert a["u"] == pytest.approx(40 / 60)
    assert a["beta_dedup"] == pytest.approx(40 / 6)
    assert a["beta_slot"] == pytest.approx(60 / 4)
    assert a["r"] == pytest.approx((40 / 6) / 15)
    assert a["saving"] == pytest.approx((1.0 - 3.0) / 2)


def test_sign_robustness_threshold():
    eps = 0.1
    edge = math.log((1 + eps) / (1 - eps))
    assert cm.sign_is_robust(1.0, math.exp(-edge * 1.01), eps)
    assert not cm.sign_is_robust(1.0, math.exp(-edge * 0.99), eps)


def test_crossover_first_positive_saving():
    assert cm.crossover([1, 2, 3, 4], [-1.0, -0.2, 0.3, 0.5]) == 3
    assert cm.crossover([2, 8], [-1.0, -0.5]) is None


def test_fits_recover_known_parameters():
    beta, t0 = 5e12, 3e-6
    b = np.linspace(1e8, 6e8, 9)
    fb, ft = cm.fit_bandwidth(b, b / beta + t0)
    assert fb == pytest.approx(beta, rel=1e-9) and ft == pytest.approx(t0, rel=1e-6)
    U = np.array([8, 12, 20, 31, 9, 15])
    nm = np.array([8, 16, 32, 64, 16, 64])
    be = 12.58e6
    c_u, c_re = 1 / 5e12, 0.2 / 5e12
    t = 2e-6 + be * (c_u * U + c_re * (nm - U))
    f = cm.fit_reread(U, nm, be, t)
    assert f["reread_cost"] == pytest.approx(0.2, rel=1e-6)
    assert f["t0"] == pytest.approx(2e-6, rel=1e-6)
