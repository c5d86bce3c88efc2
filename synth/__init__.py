"""Seeded synthetic inputs shared by the oracle and the GPU path (no method arithmetic)."""
from .configs import ALL, BY_NAME, BF16, F32, FP8, LayerConfig  # noqa: F401
from .gen import Case, make_case, expert_weights, stack_experts  # noqa: F401
