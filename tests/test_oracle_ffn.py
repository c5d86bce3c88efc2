"""Pins of the oracle's expert FFN (SwiGLU), dedup/per-slot modes, combine and bytes.

References: torch's SiLU and linear layers (library routines the oracle does
not call), the identity-weight special case that reduces SwiGLU to the
textbook silu(c x) * x, single-nonzero weights that pin each matrix's stored
orientation, and the expert sizes the pages print.

Mode equality follows the expert-bytes page (abstract): the deduplicating
kernel reads each selected expert once per pass and the per-slot kernel once
per token, for the same result.  Combine is the weighted sum of the adaptive
verification page, Sec. 2.2.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synth import make_case
from synth.configs import DSV2LITE, OLMOE, TINY, LayerConfig

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _stored_f32(wg, wu, wd):
    return {"w_gate": wg.astype(np.float32), "w_up": wu.astype(np.float32),
            "w_down": wd.astype(np.float32)}


def _torch_swiglu(x, wg, wu, wd):
    xt = torch.from_numpy(x.astype(np.float64))
    a = torch.nn.functional.linear(xt, torch.from_numpy(wg.astype(np.float64)))
    v = torch.nn.functional.linear(xt, torch.from_numpy(wu.astype(np.float64)))
    h = torch.nn.functional.silu(a) * v
    return torch.nn.functional.linear(h, torch.from_numpy(wd.astype(np.float64))).numpy()


@pytest.mark.parametrize("d,f", [(8, 12), (16, 4), (32, 32)])
def test_swiglu_matches_torch_linear_layers(d, f):
    g = np.random.default_rng(d * f)
    wg, wu = g.standard_normal((f, d)).astype(np.float32), g.standard_normal((f, d)).astype(np.float32)
    wd = g.standard_normal((d, f)).astype(np.float32)
    x = g.standard_normal(d)
    ex = oracle.DecodedExpert(_stored_f32(wg, wu, wd), "f32")
    assert np.allclose(oracle.swiglu(x, ex), _torch_swiglu(x, wg, wu, wd), rtol=1e-12, atol=1e-12)


def test_identity_weights_reduce_to_textbook_silu():
    d = 16
    c = 0.75
    x = np.linspace(-4, 4, d)
    eye = np.eye(d, dtype=np.float32)
    ex = oracle.DecodedExpert(_stored_f32(c * eye, eye, eye), "f32")
    ref = torch.nn.functional.silu(torch.from_numpy(c * x)).numpy() * x
    assert np.allclose(oracle.swiglu(x, ex), ref, rtol=1e-14, atol=1e-14)


def test_zero_gate_gives_zero_output():
    g = np.random.default_rng(2)
    d, f = 8, 6
    ex = oracle.DecodedExpert(_stored_f32(np.zeros((f, d)), g.standard_normal((f, d)),
                                          g.standard_normal((d, f))), "f32")
    assert np.all(oracle.swiglu(g.standard_normal(d), ex) == 0.0)


def test_single_nonzero_weights_pin_stored_orientation():
    d, f = 5, 3
    i0, j0, c0 = 4, 2, 1
    alpha, gv, uv, wv = 1.5, 0.5, -2.0, 3.0
    wg = np.zeros((f, d)); wg[j0, i0] = gv     # gate/up stored [f][d]
    wu = np.zeros((f, d)); wu[j0, i0] = uv
    wd = np.zeros((d, f)); wd[c0, j0] = wv     # down stored [d][f]
    x = np.zeros(d); x[i0] = alpha
    y = oracle.swiglu(x, oracle.DecodedExpert(_stored_f32(wg, wu, wd), "f32"))
    a = torch.tensor(gv * alpha, dtype=torch.float64)
    expect = wv * float(torch.nn.functional.silu(a)) * (uv * alpha)
    assert y[c0] == pytest.approx(expect, rel=1e-15)
    assert np.count_nonzero(y) == 1


def test_permuting_intermediate_axis_leaves_output_unchanged():
    g = np.random.default_rng(5)
    d, f = 6, 10
    wg, wu, wd = g.standard_normal((f, d)), g.standard_normal((f, d)), g.standard_normal((d, f))
    x = g.standard_normal(d)
    p = g.permutation(f)
    y0 = oracle.swiglu(x, oracle.DecodedExpert(_stored_f32(wg, wu, wd), "f32"))
    y1 = oracle.swiglu(x, oracle.DecodedExpert(_stored_f32(wg[p], wu[p], wd[:, p]), "f32"))
    assert np.allclose(y0, y1, rtol=1e-12, atol=1e-12)


def test_down_projection_is_linear():
    g = np.random.default_rng(6)
    d, f = 6, 10
    wg, wu, wd = g.standard_normal((f, d)), g.standard_normal((f, d)), g.standard_normal((d, f))
    x = g.standard_normal(d)
    y1 = oracle.swiglu(x, oracle.DecodedExpert(_stored_f32(wg, wu, wd), "f32"))
    y2 = oracle.swiglu(x, oracle.DecodedExpert(_stored_f32(wg, wu, 2 * wd), "f32"))
    assert np.allclose(y2, 2 * y1, rtol=1e-6)


# --------------------------------------------------------------- the two modes
SMALL_SHARED = LayerConfig(name="small_shared", cfg_id=90, E=12, K=3, d=32, f=48, S=2,
                           w_dtype="bf16", x_dtype="bf16", n_values=(5,),
                           routing=("markov:0.5",), tolerance=1e-2)
SMALL_FP8 = LayerConfig(name="small_fp8", cfg_id=91, E=6, K=2, d=256, f=128, S=0,
                        w_dtype="fp8_e4m3", x_dtype="bf16", n_values=(3,),
                        routing=("iid",), tolerance=3e-2)


@pytest.mark.parametrize("cfg,n,routing,tree", [
    (TINY, 4, None, False), (SMALL_SHARED, 5, "markov:0.5", False),
    (SMALL_SHARED, 7, "markov:0.8", True), (SMALL_FP8, 3, "iid", False),
])
def test_dedup_equals_perslot_bit_for_bit(cfg, n, routing, tree):
    case = make_case(cfg, n, routing, seed=3, tree=tree)
    a = oracle.verify_op(case, "dedup")
    b = oracle.verify_op(case, "perslot")
    assert np.array_equal(a["y_slots"], b["y_slots"])
    assert np.array_equal(a["y_shared"], b["y_shared"])
    assert np.array_equal(a["out"], b["out"])
    # each mode's own read counter equals the byte formula of its mode
    b_e = oracle.expert_bytes(cfg.d, cfg.f, cfg.w_dtype)
    assert a["bytes_read"] == (a["union"]["U"] + cfg.S) * b_e == a["union_bytes"]
    assert b["bytes_read"] == n * (cfg.K + cfg.S) * b_e == b["requested_bytes"]


@pytest.mark.parametrize("cfg", [TINY, SMALL_SHARED])
def test_one_token_is_K_single_expert_evaluations(cfg):
    case = make_case(cfg, 1, None, seed=11)
    r = oracle.verify_op(case, "dedup")
    assert r["union"]["U"] == cfg.K
    assert r["union_bytes"] == r["requested_bytes"]  # u = 1 at n = 1
    x = oracle.decode_x(case.x, cfg.x_dtype)[0]
    ref = np.zeros(cfg.d)
    for k in range(cfg.K):
        ex = oracle.DecodedExpert(case.expert(int(r["ids"][0, k])), cfg.w_dtype)
        ref += r["gates"][0, k] * oracle.swiglu(x, ex)
    for s in range(cfg.S):
        ref += oracle.swiglu(x, oracle.DecodedExpert(case.shared(s), cfg.w_dtype))
    assert np.allclose(r["out"][0], ref, rtol=1e-12, atol=1e-12)


def test_shared_outputs_do_not_depend_on_routing():
    c1 = make_case(SMALL_SHARED, 4, "markov:0.0", seed=1)
    c2 = make_case(SMALL_SHARED, 4, "markov:0.8", seed=1)
    assert np.array_equal(c1.x, c2.x)
    r1, r2 = oracle.verify_op(c1), oracle.verify_op(c2)
    assert not np.array_equal(r1["ids"], r2["ids"])
    assert np.array_equal(r1["y_shared"], r2["y_shared"])


def test_combine_one_hot_and_uniform_gates():
    g = np.random.default_rng(9)
    y = g.standard_normal((3, 4, 7))
    gates = np.zeros((3, 4)); gates[:, 2] = 1.0
    assert np.array_equal(oracle.combine(y, gates, None), y[:, 2])
    same = np.repeat(y[:, :1], 4, axis=1)
    w = g.random((3, 4)); w /= w.sum(axis=1, keepdims=True)
    assert np.allclose(oracle.combine(same, w, None), y[:, 0], rtol=1e-13, atol=1e-13)
    sh = g.standard_normal((3, 2, 7))
    assert np.allclose(oracle.combine(y, gates, sh), y[:, 2] + sh.sum(axis=1), rtol=1e-14)


# ----------------------------------------------------------------------- bytes
def test_expert_sizes_printed_on_the_pages():
    with open(os.path.join(GOLDEN, "expert_sizes.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        b = oracle.expert_bytes(c["d"], c["f"], c["w_dtype"])
        if c["w_dtype"] == "fp8_e4m3" and not c["scales_included"]:
            b -= 3 * (c["d"] // 128) * (c["f"] // 128) * 4
        assert round(b / 1e6, c["decimals"]) == c["megabytes"], c["name"]


def test_byte_counts_bracket():
    # union bytes lie between one pass over K experts and the per-slot request
    for n in (1, 2, 8):
        for U in range(OLMOE.K, min(n * OLMOE.K, OLMOE.E) + 1):
            ub, rb = oracle.byte_counts(OLMOE.d, OLMOE.f, "bf16", OLMOE.K, 0, n, U)
            assert ub <= rb and ub * n >= rb
    ub, rb = oracle.byte_counts(DSV2LITE.d, DSV2LITE.f, "bf16", DSV2LITE.K, 2, 4, 10)
    b = oracle.expert_bytes(DSV2LITE.d, DSV2LITE.f, "bf16")
    assert (ub, rb) == (12 * b, 4 * 8 * b)
