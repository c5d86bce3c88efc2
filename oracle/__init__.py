"""CPU oracle of the MoE verify-pass expert operation (float64 numpy).

TEST INFRASTRUCTURE ONLY: used by tests/, the graft entry point's smoke check
and the cpu_baseline leg of bench.py; never by the product path.  Shares no
code with the HIP library.
"""
from .moe_ref import (  # noqa: F401
    DecodedExpert, build_union, byte_counts, combine, decode_bf16, decode_fp8_e4m3fn,
    decode_matrix, decode_x, distinct_share, expert_bytes, ffn_dedup, ffn_perslot,
    reuse_last, route_topk, silu, swiglu, union_size, verify_op,
)
from .evict_ref import evict_select, is_ancestor_closed, path_scores, rank_nodes  # noqa: F401,E402
from .ecospec_ref import (  # noqa: F401,E402
    cumulative_probability, ecospec_select, path_footprints,
)
from .budget_ref import apply_budget, expert_scores, kept_experts, verify_op_budget  # noqa: F401,E402
from .bellman_ref import accept_probs, bellman_policy, expected_cost  # noqa: F401,E402
