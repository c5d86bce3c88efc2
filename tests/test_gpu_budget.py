"""GPU parity of the per-layer expert budget ("MoE-Spec: Expert Budgeting for
Efficient Speculative Decoding", abstract) against the oracle, through the C
ABI.

- moe_expert_budget on caller-given ids and float32 gates: the budgeted union
  arrays bit for bit, the gates exactly (renorm 0: copied or zeroed) or
  within float32 division rounding (renorm 1).  The device sums the gates in
  float32, the oracle the same values in float64: ties of equal gates are
  exact in both, and every other case first checks that no two
  contributions near the cut lie closer than float32 summation could move
  them.
- the whole budgeted pass (route, union, budget, deduplicating FFN, combine)
  against the oracle's: routing and budgeted union bit for bit, expert and
  layer outputs within the tolerances of ``gpu_harness``, dropped slots'
  output rows exactly zero; the router's gates come from each side's own
  softmax, so every case first checks that no two contributions near the cut
  lie closer than their float32 rounding could move them (else the inputs
  would have two valid kept sets).
- moe_verify_layer_budget against that chain of entry points: every output
  bit for bit, on two calls in a row.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.budget_ref import apply_budget, verify_op_budget
from synth import make_case
from synth.configs import DSV2LITE, LayerConfig, OLMOE, TINY

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU machines, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from moe_speculative_decoding_amd import _lib as L  # noqa: E402
from moe_speculative_decoding_amd.layer import (  # noqa: E402
    VerifyBuffers, to_device, verify_layer_budget, verify_pass_budget)
from gpu_harness import DEV, _bits, check_vectors, derived_bound, upload_layer  # noqa: E402

RAGGED_BF16 = LayerConfig(name="ragged_bf16", cfg_id=80, E=16, K=4, d=264, f=136, S=1,
                          w_dtype="bf16", x_dtype="bf16", n_values=(1, 5, 32),
                          routing=("markov:0.8",), tolerance=1e-2)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _gpu_budget(ids, gates32, E, C, renorm):
    n, K = ids.shape
    cap = min(n * K, E)
    i32 = dict(dtype=torch.int32, device=DEV)
    U = torch.zeros(1, **i32)
    union_ids = torch.full((cap,), -9, **i32)
    offsets = torch.full((cap + 1,), -9, **i32)
    perm = torch.full((n * K,), -9, **i32)
    slot_rank = torch.full((n * K,), -9, **i32)
    g = dev(gates32)
    gout = torch.full((n, K), -5.0, dtype=torch.float32, device=DEV)
    d_ids = dev(ids)
    L.moe_build_union(d_ids, n, K, E, U, union_ids, offsets, perm, slot_rank)
    L.moe_expert_budget(g, n, K, E, C, renorm, U, union_ids, offsets, perm, slot_rank, gout)
    torch.cuda.synchronize()
    return {"U": int(U.item()), "union_ids": union_ids.cpu().numpy(),
            "offsets": offsets.cpu().numpy(), "perm": perm.cpu().numpy(),
            "slot_rank": slot_rank.cpu().numpy(), "gates": gout.cpu().numpy()}


def _routing(seed, n, K, E, pool=None, equal=False):
    g = np.random.default_rng(seed)
    pool = E if pool is None else pool
    ids = np.stack([g.choice(pool, size=K, replace=False) for _ in range(n)]).astype(np.int32)
    raw = np.full((n, K), 1.0) if equal else g.random((n, K)) + 0.05
    gates = (raw / raw.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, gates


@pytest.mark.parametrize("n,K,E,pool,C,renorm,equal", [
    (4, 2, 8, None, 3, 0, False), (4, 2, 8, None, 3, 1, False),
    (8, 8, 64, None, 16, 0, False), (8, 8, 64, None, 16, 1, False),
    (8, 8, 64, 20, 5, 1, False),                   # heavy reuse: few, large groups
    (32, 8, 256, None, 100, 1, False),             # 256 slots, union near 256
    (32, 8, 256, None, 1, 0, False),
    (16, 4, 32, None, 7, 0, True),                 # equal gates: ties go to the lower id
    (5, 3, 9, None, 50, 1, False),                 # budget not binding: nothing changes
    (1, 8, 64, None, 3, 1, False),
])
def test_expert_budget_matches_oracle(n, K, E, pool, C, renorm, equal):
    ids, g32 = _routing(1000 + n * 7 + C, n, K, E, pool, equal)
    print("budget n=%d K=%d E=%d C=%d renorm=%d" % (n, K, E, C, renorm), flush=True)
    un = oracle.build_union(ids, E)
    ref = apply_budget(ids, g32.astype(np.float64), un, C, bool(renorm))
    assert equal or _margin_ok({"union": ref}, C, n), "near-tie at the cut: pick another seed"
    got = _gpu_budget(ids, g32, E, C, renorm)
    assert got["U"] == ref["U"] == min(C, un["U"])
    for key in ("union_ids", "offsets", "perm", "slot_rank"):
        assert np.array_equal(got[key], ref[key]), key
    if renorm:
        assert np.all(np.abs(got["gates"] - ref["gates"]) <= 2e-7 * np.abs(ref["gates"]))
        assert np.array_equal(got["gates"] == 0.0, ref["gates"] == 0.0)
    else:
        assert np.array_equal(got["gates"].astype(np.float64), ref["gates"])


def _margin_ok(ref, C, n):
    """No contribution within float32 reach of the cut (see the module docstring)."""
    sc = np.sort(ref["union"]["scores"].astype(np.float64))[::-1]
    if C >= len(sc):
        return True
    return sc[C - 1] - sc[C] > 1e-5 * n


@pytest.mark.parametrize("cfg,n,routing,tree,C,renorm", [
    (TINY, 4, None, False, 3, 0),
    (RAGGED_BF16, 5, None, False, 4, 1),
    (RAGGED_BF16, 32, None, True, 6, 0),
    (DSV2LITE, 5, "markov:0.5", False, 6, 1),
    (OLMOE, 8, "markov:0.5", False, 16, 0),
    (OLMOE, 8, "markov:0.0", False, 24, 1),
    (OLMOE, 1, "markov:0.5", False, 3, 1),        # one token: its top-3 with renormalised gates
])
def test_budgeted_pass_matches_oracle(cfg, n, routing, tree, C, renorm):
    case = make_case(cfg, n, routing, seed=3, tree=tree)
    ref = verify_op_budget(case, C, bool(renorm))
    assert _margin_ok(ref, C, n), "inputs with a near-tie at the cut: pick another seed"
    bud = ref["union"]
    U = bud["U"]
    assert U == min(C, bud["U_before"])
    layer = upload_layer(case, bud["kept"])
    x, logits = to_device(case.x, DEV), to_device(case.logits, DEV)
    tight = min(cfg.tolerance, derived_bound(cfg))
    chain = VerifyBuffers(layer, n, DEV)
    chain.y_slots.fill_(3.0)   # dropped rows must come back zero
    print("budget pass %s n=%d C=%d renorm=%d" % (cfg.name, n, C, renorm), flush=True)
    verify_pass_budget(layer, chain, x, logits, n, C, bool(renorm))
    torch.cuda.synchronize()
    assert L.moe_get_error(chain.ws) == L.MOE_OK
    assert np.array_equal(chain.ids[:n].cpu().numpy(), ref["ids"])
    gates = chain.gates[:n].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(gates - ref["gates"]) <= 1e-6 + 1e-5 * np.abs(ref["gates"])), "gates"
    assert int(chain.U.item()) == U
    for key in ("union_ids", "offsets"):
        got = getattr(chain, key).cpu().numpy()[:len(bud[key])]
        assert np.array_equal(got, bud[key]), key
    assert np.array_equal(chain.perm[:n * cfg.K].cpu().numpy(), bud["perm"])
    assert np.array_equal(chain.slot_rank[:n * cfg.K].cpu().numpy(), bud["slot_rank"])
    b = chain.bytes.cpu().numpy()
    assert int(b[0]) == ref["union_bytes"] and int(b[1]) == ref["requested_bytes"]
    y = chain.y_slots[:n].cpu().numpy()
    keep = bud["slot_rank"].reshape(n, cfg.K) >= 0
    assert np.all(y[~keep] == 0.0), "dropped slots must have zero rows"
    check_vectors(y[keep], ref["y_slots"][keep], tight, "budget y_slots")
    if cfg.S:
        check_vectors(chain.y_shared[:n, :cfg.S].cpu().numpy(), ref["y_shared"], tight,
                      "budget y_shared")
    check_vectors(chain.out[:n].float().cpu().numpy(), ref["out"], tight, "budget out")

    # one launch: the chain bit for bit, twice in a row on one workspace
    buf = VerifyBuffers(layer, n, DEV)
    for call in range(2):
        print("  fused budget call %d" % call, flush=True)
        buf.out.zero_()
        buf.y_slots.fill_(5.0)
        verify_layer_budget(layer, buf, x, logits, n, C, bool(renorm))
        torch.cuda.synchronize()
        assert L.moe_get_error(buf.ws) == L.MOE_OK
        pairs = [("ids", buf.ids[:n], chain.ids[:n]), ("gates", buf.gates[:n], chain.gates[:n]),
                 ("bytes", buf.bytes, chain.bytes), ("y_slots", buf.y_slots[:n], chain.y_slots[:n]),
                 ("out", buf.out[:n], chain.out[:n]), ("U", buf.U, chain.U),
                 ("union_ids", buf.union_ids, chain.union_ids),
                 ("offsets", buf.offsets, chain.offsets),
                 ("perm", buf.perm[:n * cfg.K], chain.perm[:n * cfg.K]),
                 ("slot_rank", buf.slot_rank[:n * cfg.K], chain.slot_rank[:n * cfg.K])]
        if cfg.S:
            pairs.append(("y_shared", buf.y_shared[:n, :cfg.S], chain.y_shared[:n, :cfg.S]))
        for name, a, bb in pairs:
            assert np.array_equal(_bits(a), _bits(bb)), "fused budget call %d: %s" % (call, name)
    buf.out.zero_()
    verify_layer_budget(layer, buf, x, logits, n, C, bool(renorm), keep=False)
    torch.cuda.synchronize()
    assert L.moe_get_error(buf.ws) == L.MOE_OK
    assert np.array_equal(_bits(buf.out[:n]), _bits(chain.out[:n])), "fused (workspace outputs)"
