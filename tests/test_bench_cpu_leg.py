"""The CPU baseline of bench.py times the oracle itself: its thread-pool split
(one oracle call per union expert, slot or set of shared experts, rows copied
into place) must compute the same layer output, bit for bit, as one oracle
call for the whole pass, and read exactly the bytes the pass defines (union
bytes for deduplication, requested bytes per slot).  Small shapes, CPU only.
"""
from dataclasses import replace

import numpy as np
import pytest

import bench
import oracle
from synth import make_case
from synth.configs import BF16, TINY

# a bf16 shape with two shared experts, small enough for the CPU suite
SMALL_SHARED = replace(TINY, name="tiny-shared", cfg_id=91, E=16, K=4, d=256, f=384, S=2,
                       w_dtype=BF16, x_dtype=BF16, routing=("markov:0.5",))


@pytest.mark.parametrize("cfg,n,routing", [
    (TINY, 4, "logits_iid"),
    (SMALL_SHARED, 1, "markov:0.5"),
    (SMALL_SHARED, 5, "markov:0.5"),
])
@pytest.mark.parametrize("mode", ["dedup", "perslot"])
def test_pooled_oracle_pass_matches_single_call(monkeypatch, cfg, n, routing, mode):
    outs = []
    combine = oracle.combine

    def spy(y, gates, ysh):
        out = combine(y, gates, ysh)
        outs.append(out)
        return out

    monkeypatch.setattr(oracle, "combine", spy)
    case = make_case(cfg, n, routing, seed=0, window=0, layer=0)
    _, read1, ev1 = bench._oracle_pass(cfg, case, mode, 1, 64)
    _, read4, ev4 = bench._oracle_pass(cfg, case, mode, 4, 64)
    assert len(outs) == 2 and np.array_equal(outs[0], outs[1])

    ids, _ = oracle.route_topk(case.logits, cfg.K)
    U = oracle.build_union(ids, cfg.E)["U"]
    ub, rb = oracle.byte_counts(cfg.d, cfg.f, cfg.w_dtype, cfg.K, cfg.S, n, U)
    want = ub if mode == "dedup" else rb
    assert read1 == read4 == want
    assert ev1 == ev4 == (U + cfg.S if mode == "dedup" else n * (cfg.K + cfg.S))
    # and the pass is the oracle's verify op
    ref = oracle.verify_op(case, mode)
    assert np.array_equal(outs[0], ref["out"])
