"""GPU parity of the HIP path against the oracle, through the C ABI.

Routing, union and permutation are compared bit for bit; expert outputs and
the combined layer output within the tolerances of ``gpu_harness``.  Cases:
the five layer shapes at their real sizes (the DeepSeek-V3 shape at its
smallest pass sizes), plus small shapes with ragged tails (d, f not
multiples of a load step or of a workgroup's row block), groups of more
tokens than one LDS tile holds, K = E, ties and NaN logits, and invalid ids.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import make_case
from synth.configs import DSV2LITE, DSV3, LayerConfig, OLMOE, QWEN3, TINY

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from moe_speculative_decoding_amd import _lib as L  # noqa: E402
from gpu_harness import DEV, run_case  # noqa: E402


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


# ------------------------------------------------------------ fp8 decoding
def test_decode_fp8_every_code_every_byte_position():
    codes = np.concatenate([np.arange(256, dtype=np.uint8)] * 4 + [np.arange(3, dtype=np.uint8)])
    # shift so each code lands in every position of its dword
    codes = np.concatenate([codes[1:], codes[:1]])
    out = torch.empty(len(codes), dtype=torch.float32, device=DEV)
    L.moe_decode_fp8(dev(codes), out, len(codes))
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.decode_fp8_e4m3fn(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


# --------------------------------------------------------------- top-K
def _route(logits, K):
    n, E = logits.shape
    ids = torch.full((n, K), -7, dtype=torch.int32, device=DEV)
    gates = torch.zeros(n, K, dtype=torch.float32, device=DEV)
    L.moe_route_topk(dev(logits), n, E, K, ids, gates)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), gates.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("cfg,n,routing,tree", [
    (TINY, 4, None, False), (QWEN3, 8, None, False), (OLMOE, 8, "markov:0.5", False),
    (DSV3, 8, "iid", False), (DSV3, 32, "markov:0.5", True), (DSV2LITE, 16, "markov:0.5", True),
])
def test_route_topk_matches_oracle(cfg, n, routing, tree):
    case = make_case(cfg, n, routing, seed=0, tree=tree)
    ids, gates = _route(case.logits, cfg.K)
    rid, rg = oracle.route_topk(case.logits, cfg.K)
    assert np.array_equal(ids, rid)
    assert np.all(np.abs(gates - rg) <= 1e-6 + 1e-5 * np.abs(rg))


@pytest.mark.parametrize("n,E,K", [(32, 256, 8), (5, 8, 8), (7, 13, 3), (1, 64, 1), (9, 64, 8),
                                   (3, 37, 5), (6, 100, 7)])
def test_route_topk_ties_nan_signed_zero(n, E, K):
    g = np.random.default_rng(E * 7 + K)
    vals = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, np.nan, -np.inf], dtype=np.float32)
    logits = vals[g.integers(0, len(vals), (n, E))]
    ids, _ = _route(logits, K)
    rid, _ = oracle.route_topk(logits, K)
    assert np.array_equal(ids, rid)


# --------------------------------------------------------------- union
def _union(ids, E):
    n, K = ids.shape
    cap = min(n * K, E)
    U = torch.full((1,), -9, dtype=torch.int32, device=DEV)
    uid = torch.full((cap,), -9, dtype=torch.int32, device=DEV)
    off = torch.full((cap + 1,), -9, dtype=torch.int32, device=DEV)
    perm = torch.full((n * K,), -9, dtype=torch.int32, device=DEV)
    rank = torch.full((n * K,), -9, dtype=torch.int32, device=DEV)
    L.moe_build_union(dev(ids.astype(np.int32)), n, K, E, U, uid, off, perm, rank)
    torch.cuda.synchronize()
    return {"U": int(U.item()), "union_ids": uid.cpu().numpy(), "offsets": off.cpu().numpy(),
            "perm": perm.cpu().numpy(), "slot_rank": rank.cpu().numpy()}


@pytest.mark.parametrize("n,E,K,pool", [(32, 256, 8, 256), (32, 256, 8, 12), (8, 64, 8, 64),
                                        (4, 8, 2, 8), (1, 8, 8, 8), (32, 8, 8, 8), (17, 100, 5, 9),
                                        (16, 64, 6, 64)])
def test_build_union_bit_exact(n, E, K, pool):
    g = np.random.default_rng(n * 31 + E + pool)
    for rep in range(4):
        # distinct ids per token drawn from a small subset -> heavy repetition across tokens
        subset = g.choice(E, pool, replace=False)
        ids = np.stack([g.choice(subset, K, replace=False) for _ in range(n)]).astype(np.int32)
        got = _union(ids, E)
        ref = oracle.build_union(ids, E)
        for k in ("U", "union_ids", "offsets", "perm", "slot_rank"):
            assert np.array_equal(np.asarray(got[k]), np.asarray(ref[k])), (k, rep)


@pytest.mark.parametrize("cfg,n,routing,tree", [
    (TINY, 4, None, False), (QWEN3, 8, None, False), (OLMOE, 1, "markov:0.5", False),
    (DSV3, 32, "markov:0.5", True), (DSV3, 32, "iid", True), (DSV2LITE, 16, "markov:0.8", True),
])
def test_route_union_fused_matches_oracle(cfg, n, routing, tree):
    case = make_case(cfg, n, routing, seed=4, tree=tree)
    E, K = cfg.E, cfg.K
    cap = min(n * K, E)
    out = {k: torch.full((m,), -9, dtype=torch.int32, device=DEV) for k, m in
           (("ids", n * K), ("U", 1), ("union_ids", cap), ("offsets", cap + 1), ("perm", n * K),
            ("slot_rank", n * K))}
    gates = torch.zeros(n * K, dtype=torch.float32, device=DEV)
    L.moe_route_union(dev(case.logits), n, E, K, out["ids"], gates, out["U"], out["union_ids"],
                      out["offsets"], out["perm"], out["slot_rank"])
    torch.cuda.synchronize()
    rid, rg = oracle.route_topk(case.logits, K)
    assert np.array_equal(out["ids"].cpu().numpy().reshape(n, K), rid)
    g = gates.cpu().numpy().astype(np.float64).reshape(n, K)
    assert np.all(np.abs(g - rg) <= 1e-6 + 1e-5 * np.abs(rg))
    ref = oracle.build_union(rid, E)
    assert int(out["U"].item()) == ref["U"]
    for k in ("union_ids", "offsets", "perm", "slot_rank"):
        assert np.array_equal(out[k].cpu().numpy(), ref[k]), k


def test_route_union_with_ties_and_nan():
    g = np.random.default_rng(77)
    vals = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, np.nan], dtype=np.float32)
    for n, E, K in ((32, 256, 8), (9, 8, 8), (32, 12, 4)):
        logits = vals[g.integers(0, len(vals), (n, E))]
        cap = min(n * K, E)
        ids = torch.empty(n * K, dtype=torch.int32, device=DEV)
        gates = torch.empty(n * K, dtype=torch.float32, device=DEV)
        U = torch.empty(1, dtype=torch.int32, device=DEV)
        uid = torch.empty(cap, dtype=torch.int32, device=DEV)
        off = torch.empty(cap + 1, dtype=torch.int32, device=DEV)
        perm = torch.empty(n * K, dtype=torch.int32, device=DEV)
        rank = torch.empty(n * K, dtype=torch.int32, device=DEV)
        L.moe_route_union(dev(logits), n, E, K, ids, gates, U, uid, off, perm, rank)
        torch.cuda.synchronize()
        rid, _ = oracle.route_topk(logits, K)
        assert np.array_equal(ids.cpu().numpy().reshape(n, K), rid)
        ref = oracle.build_union(rid, E)
        assert int(U.item()) == ref["U"]
        assert np.array_equal(perm.cpu().numpy(), ref["perm"])
        assert np.array_equal(off.cpu().numpy(), ref["offsets"])


def test_build_union_flags_out_of_range_ids():
    ids = np.array([[0, 3], [8, 1]], dtype=np.int32)
    assert _union(ids, 8)["U"] == -1
    ids = np.array([[0, -1]], dtype=np.int32)
    assert _union(ids, 8)["U"] == -1


# ----------------------------------------------------------- expert FFN
RAGGED_BF16 = LayerConfig(name="ragged_bf16", cfg_id=80, E=16, K=4, d=264, f=136, S=1,
                          w_dtype="bf16", x_dtype="bf16", n_values=(1, 5, 32),
                          routing=("markov:0.8",), tolerance=1e-2)
RAGGED_FP8 = LayerConfig(name="ragged_fp8", cfg_id=81, E=8, K=2, d=384, f=256, S=1,
                         w_dtype="fp8_e4m3", x_dtype="bf16", n_values=(3, 9),
                         routing=("markov:0.5",), tolerance=3e-2)
RAGGED_F32 = LayerConfig(name="ragged_f32", cfg_id=82, E=6, K=3, d=300, f=68, S=2,
                         w_dtype="f32", x_dtype="f32", n_values=(2, 11),
                         routing=("markov:0.5",), tolerance=1e-5)


@pytest.mark.parametrize("cfg,n,routing,tree", [
    (TINY, 4, None, False),
    (RAGGED_BF16, 1, None, False), (RAGGED_BF16, 5, None, False), (RAGGED_BF16, 32, None, True),
    (RAGGED_BF16, 32, "markov:1.0", False),
    (RAGGED_FP8, 3, None, False), (RAGGED_FP8, 9, None, False),
    (RAGGED_F32, 2, None, False), (RAGGED_F32, 11, None, False),
])
def test_ffn_small_and_ragged(cfg, n, routing, tree):
    case = make_case(cfg, n, routing, seed=2, tree=tree)
    run_case(case)


@pytest.mark.parametrize("n,p", [(1, 0.5), (2, 0.5), (4, 0.5), (8, 0.5), (8, 0.0), (8, 0.8)])
def test_ffn_olmoe_shape(n, p):
    run_case(make_case(OLMOE, n, "markov:%s" % p, seed=0))


@pytest.mark.parametrize("n", [1, 5, 8])
def test_ffn_qwen3_shape(n):
    run_case(make_case(QWEN3, n, None, seed=1))


@pytest.mark.parametrize("n,tree", [(3, False), (8, False), (16, True)])
def test_ffn_dsv2lite_shape(n, tree):
    run_case(make_case(DSV2LITE, n, "markov:0.5", seed=0, tree=tree))


@pytest.mark.parametrize("n,routing", [(1, "iid"), (2, "markov:0.5"), (6, "markov:0.5")])
def test_ffn_dsv3_shape(n, routing):
    run_case(make_case(DSV3, n, routing, seed=0))


# the DeepSeek-V3 expert shape with 16 experts, so a 32-node tree puts up to
# 32 tokens on one expert (8 token tiles in the up phase, 4 in the down phase)
DSV3_E16 = LayerConfig(name="dsv3_e16", cfg_id=83, E=16, K=8, d=7168, f=2048, S=0,
                       w_dtype="fp8_e4m3", x_dtype="bf16", n_values=(32,),
                       routing=("markov:0.5",), tolerance=3e-2)


def test_ffn_dsv3_expert_shape_tree32():
    run_case(make_case(DSV3_E16, 32, "markov:0.5", seed=0, tree=True))


# 32 tokens on the fp8 path whose union holds groups of 12 and 10 tokens and
# many of 1-8: the one-launch pass splits its ranges by cost (the two large
# groups exceed the 8-token UP tile and take the general path, one pass per
# tile), and its DOWN phase runs the 16-token tile although the pass is
# compiled for 32; the chain of entry points runs the 32-token DOWN tile, and
# the two must agree bit for bit (run_case) and with the oracle
FP8_SMALL = LayerConfig(name="fp8_small", cfg_id=84, E=32, K=4, d=512, f=256, S=0,
                        w_dtype="fp8_e4m3", x_dtype="bf16", n_values=(32,),
                        routing=("iid",), tolerance=3e-2)


def test_ffn_fp8_groups_beyond_the_up_tile():
    import dataclasses
    case = make_case(FP8_SMALL, 32, "iid", seed=3)
    lg = case.logits.copy()
    lg[:, 0] = -10.0
    lg[:, 1] = -10.0
    lg[:12, 0] = 10.0
    lg[12:22, 1] = 10.0
    case = dataclasses.replace(case, logits=lg)
    ref = oracle.verify_op(case, "dedup")
    un = ref["union"]
    counts = np.diff(np.asarray(un["offsets"][:int(un["U"]) + 1]))
    assert counts.max() == 12 and sorted(counts)[-2] == 10
    run_case(case, ref=ref)


# ------------------------------------------------------- invalid expert ids
def test_perslot_bad_id_gives_zero_row_and_error():
    from moe_speculative_decoding_amd.layer import VerifyBuffers
    from gpu_harness import upload_layer
    case = make_case(TINY, 2, None, seed=5)
    layer = upload_layer(case)
    buf = VerifyBuffers(layer, 2, DEV)
    ids = np.array([[1, 2], [3, 99]], dtype=np.int32)
    buf.y_slots.fill_(7.0)
    L.moe_expert_ffn_perslot(layer.shape, layer.weights, dev(case.x), 2, dev(ids), buf.y_slots,
                             None, buf.bytes, buf.ws, buf.ws_bytes)
    assert L.moe_get_error(buf.ws) == L.MOE_ERR_BAD_IDS
    assert L.moe_get_error(buf.ws) == L.MOE_OK  # cleared
    y = buf.y_slots.cpu().numpy()
    assert np.all(y[1, 1] == 0.0)
    assert np.all(np.isfinite(y[0])) and not np.all(y[0, 0] == 7.0)


def test_dedup_after_bad_union_reports_error():
    from moe_speculative_decoding_amd.layer import VerifyBuffers
    from gpu_harness import upload_layer
    case = make_case(TINY, 2, None, seed=5)
    layer = upload_layer(case)
    buf = VerifyBuffers(layer, 2, DEV)
    ids = dev(np.array([[1, 2], [3, -4]], dtype=np.int32))
    L.moe_build_union(ids, 2, 2, 8, buf.U, buf.union_ids, buf.offsets, buf.perm, buf.slot_rank)
    L.moe_expert_ffn_dedup(layer.shape, layer.weights, dev(case.x), 2, buf.U, buf.union_ids,
                           buf.offsets, buf.perm, buf.y_slots, None, buf.bytes, buf.ws, buf.ws_bytes)
    assert L.moe_get_error(buf.ws) == L.MOE_ERR_BAD_IDS
    assert int(buf.U.item()) == -1


def test_combine_matches_oracle_f32_and_bf16():
    g = np.random.default_rng(12)
    n, K, S, d = 7, 6, 2, 1000
    y = g.standard_normal((n, K, d)).astype(np.float32)
    gates = g.random((n, K)).astype(np.float32)
    ysh = g.standard_normal((n, S, d)).astype(np.float32)
    ref = oracle.combine(y.astype(np.float64), gates.astype(np.float64), ysh.astype(np.float64))
    out = torch.empty(n, d, dtype=torch.float32, device=DEV)
    L.moe_combine(dev(y), dev(gates), dev(ysh), n, K, S, d, out, L.MOE_F32)
    got = out.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-5 * (1 + np.max(np.abs(ref)))
    outb = torch.empty(n, d, dtype=torch.bfloat16, device=DEV)
    L.moe_combine(dev(y), dev(gates), dev(ysh), n, K, S, d, outb, L.MOE_BF16)
    gotb = outb.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(gotb - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


# ------------------------------------------- one-launch pass, one workspace
def test_layer_one_workspace_across_pass_sizes():
    """moe_verify_layer on one workspace for passes of different sizes (and so
    different grids and tiles) in a row: every call matches the chain of entry
    points bit for bit (the hand-over flags of one call never satisfy the
    next call's waits)."""
    from moe_speculative_decoding_amd.layer import VerifyBuffers, to_device, verify_layer, verify_pass
    from gpu_harness import _bits, upload_layer
    cfg = RAGGED_BF16
    layer = upload_layer(make_case(cfg, 8, None, seed=9))  # every expert of the layer
    shared = VerifyBuffers(layer, 8, DEV)
    for step, n in enumerate((8, 1, 5, 2, 8, 1)):
        case = make_case(cfg, n, None, seed=20 + step)
        x, logits = to_device(case.x, DEV), to_device(case.logits, DEV)
        for mode in (L.MOE_MODE_DEDUP, L.MOE_MODE_PERSLOT):
            print("step %d n=%d mode=%d" % (step, n, mode), flush=True)
            chain = VerifyBuffers(layer, n, DEV)
            verify_pass(layer, chain, x, logits, n, mode)
            shared.out.zero_()
            verify_layer(layer, shared, x, logits, n, mode)
            torch.cuda.synchronize()
            assert L.moe_get_error(shared.ws) == L.MOE_OK
            assert np.array_equal(_bits(shared.out[:n]), _bits(chain.out[:n])), (step, n, mode)


# ------------------------------- one-launch pass: top-K of few tokens in teams
@pytest.mark.parametrize("n,E,K", [(1, 37, 5), (1, 256, 8), (2, 100, 8), (3, 256, 8),
                                   (4, 64, 8), (5, 100, 7), (6, 256, 3), (7, 64, 8)])
def test_layer_routing_teams_with_ties(n, E, K):
    """The one-launch pass splits the rank counts of each of few tokens (n <= 6)
    over a team of wavefronts: ids, union and byte counters bit for bit against
    the oracle, gates and layer output bit for bit against the chain of entry
    points (whose top-K takes one wavefront per token), with tied, NaN, -inf
    and signed-zero logits, for one, two and four experts per lane."""
    from moe_speculative_decoding_amd.layer import VerifyBuffers, to_device, verify_layer, verify_pass
    from gpu_harness import _bits, upload_layer
    cfg = LayerConfig(name="teams", cfg_id=83, E=E, K=K, d=264, f=136, S=0, w_dtype="bf16",
                      x_dtype="bf16", n_values=(n,), routing=("logits_iid",), tolerance=1e-2)
    case = make_case(cfg, n, None, seed=E + n)
    g = np.random.default_rng(1000 + 31 * E + n)
    vals = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, np.nan, -np.inf], dtype=np.float32)
    logits = vals[g.integers(0, len(vals), (n, E))]
    print("teams n=%d E=%d K=%d" % (n, E, K), flush=True)
    layer = upload_layer(case)
    x, lg = to_device(case.x, DEV), to_device(logits, DEV)
    buf = VerifyBuffers(layer, n, DEV)
    verify_layer(layer, buf, x, lg, n, L.MOE_MODE_DEDUP)
    chain = VerifyBuffers(layer, n, DEV)
    verify_pass(layer, chain, x, lg, n, L.MOE_MODE_DEDUP)
    torch.cuda.synchronize()
    assert L.moe_get_error(buf.ws) == L.MOE_OK
    rid, _ = oracle.route_topk(logits, K)
    assert np.array_equal(buf.ids[:n].cpu().numpy(), rid)
    un = oracle.build_union(rid, E)
    assert int(buf.U.item()) == un["U"]
    for k in ("union_ids", "offsets"):
        got = getattr(buf, k).cpu().numpy()[:len(un[k])]
        assert np.array_equal(got, un[k]), k
    assert np.array_equal(buf.perm[:n * K].cpu().numpy(), un["perm"])
    assert np.array_equal(buf.slot_rank[:n * K].cpu().numpy(), un["slot_rank"])
    ub, rb = oracle.byte_counts(cfg.d, cfg.f, cfg.w_dtype, K, 0, n, un["U"])
    b = buf.bytes.cpu().numpy()
    assert int(b[0]) == ub and int(b[1]) == rb
    assert np.array_equal(_bits(buf.gates[:n]), _bits(chain.gates[:n]))
    assert np.array_equal(_bits(buf.out[:n]), _bits(chain.out[:n]))


# ------------------------------------ one-launch pass, mode chosen on device
@pytest.mark.parametrize("cfg,n,routing", [(RAGGED_BF16, 5, None), (TINY, 4, None),
                                           (RAGGED_F32, 11, None), (OLMOE, 4, "markov:0.5")])
def test_layer_auto_mode_follows_eq7(cfg, n, routing):
    """moe_verify_layer_auto picks deduplication iff (U+S)/(n(K+S)) < r (the
    expert-bytes page, Eq. (7)), with the mode expected from the oracle's own
    union; its layer output matches the oracle's pass in that mode within the
    harness tolerances, its byte counters the oracle's, and (same arithmetic)
    the chain of entry points of that mode bit for bit."""
    from moe_speculative_decoding_amd.layer import (VerifyBuffers, to_device, verify_layer_auto,
                                                    verify_pass)
    from gpu_harness import _bits, check_vectors, derived_bound, upload_layer
    case = make_case(cfg, n, routing, seed=31)
    ref = oracle.verify_op(case, "dedup")
    U = int(ref["union"]["U"])
    u = (U + cfg.S) / (n * (cfg.K + cfg.S))
    refs = {L.MOE_MODE_DEDUP: ref, L.MOE_MODE_PERSLOT: oracle.verify_op(case, "perslot")}
    layer = upload_layer(case, ref["union"]["union_ids"][:U])
    x, logits = to_device(case.x, DEV), to_device(case.logits, DEV)
    chains = {}
    for mode in (L.MOE_MODE_DEDUP, L.MOE_MODE_PERSLOT):
        chains[mode] = VerifyBuffers(layer, n, DEV)
        verify_pass(layer, chains[mode], x, logits, n, mode)
    torch.cuda.synchronize()
    tight = min(cfg.tolerance, derived_bound(cfg))
    buf = VerifyBuffers(layer, n, DEV)
    mode_out = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    for r in (0.0, u * 0.999, u * 1.001, 2.0):
        expect = L.MOE_MODE_DEDUP if u < r else L.MOE_MODE_PERSLOT
        print("%s n=%d U=%d u=%.4f r=%.4f expect=%d" % (cfg.name, n, U, u, r, expect), flush=True)
        buf.out.zero_()
        verify_layer_auto(layer, buf, x, logits, n, r, mode_out)
        torch.cuda.synchronize()
        assert L.moe_get_error(buf.ws) == L.MOE_OK
        assert int(mode_out.item()) == expect
        want = refs[expect]
        check_vectors(buf.out[:n].float().cpu().numpy(), want["out"], tight, "auto out r=%g" % r)
        b = buf.bytes.cpu().numpy()
        expect0 = want["union_bytes"] if expect == L.MOE_MODE_DEDUP else want["requested_bytes"]
        assert int(b[0]) == expect0 and int(b[1]) == want["requested_bytes"], r
        chain = chains[expect]
        assert np.array_equal(_bits(buf.out[:n]), _bits(chain.out[:n])), r
