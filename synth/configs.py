"""Named shapes of the MoE expert layer that the verify-pass workloads use.

Each entry fixes the layer geometry (experts E, top-K, hidden d, expert
intermediate f, shared experts S), the storage types of weights and
activations, the pass sizes n that are exercised, and the routing recipe.
The shapes are those of public MoE checkpoints (OLMoE-1B-7B, Qwen3-30B-A3B,
DeepSeek-V2-Lite, DeepSeek-V3) as the pages name them; the values are
synthetic (see ``synth.gen``).

Pages: "Speculative Decoding for Mixture-of-Experts Models: Expert Bytes,
Kernel Bandwidth and the Best Draft Length" (abstract; Table 1 lists OLMoE,
gpt-oss, DeepSeek-V2-Lite, Qwen3); "Less Experts, Faster Decoding"
(Figure 1c: one FP8 DeepSeek-V3.1 expert is 44.04 MB).

This module holds no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

F32 = "f32"
BF16 = "bf16"
FP8 = "fp8_e4m3"

ELEM_BYTES = {F32: 4, BF16: 2, FP8: 1}


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    E: int            # routed experts
    K: int            # experts per token (the pages' m)
    d: int            # hidden size
    f: int            # expert intermediate size
    S: int            # shared experts, applied to every token with weight 1
    w_dtype: str      # expert weight storage
    x_dtype: str      # activation storage
    n_values: Tuple[int, ...]
    routing: Tuple[str, ...]          # "logits_iid", "logits_ar1", "markov:p", "iid"
    tree_nodes: Tuple[int, ...] = ()  # draft-tree sizes (heap-shaped tree)
    seeds: Tuple[int, ...] = (0,)
    tolerance: float = 1e-2           # relative L2 bound of outputs vs the oracle
    notes: str = field(default="", compare=False)

    @property
    def fp8(self) -> bool:
        return self.w_dtype == FP8


TINY = LayerConfig(
    name="tiny", cfg_id=1, E=8, K=2, d=256, f=512, S=0,
    w_dtype=F32, x_dtype=F32, n_values=(4,), routing=("logits_iid",),
    seeds=(0,), tolerance=1e-5,
    notes="x ~ N(0,1); W ~ N(0,1/d); router W_r ~ N(0,1/d); gate = softmax over top-K logits",
)

OLMOE = LayerConfig(
    name="olmoe", cfg_id=2, E=64, K=8, d=2048, f=1024, S=0,
    w_dtype=BF16, x_dtype=BF16, n_values=(1, 2, 4, 8),
    routing=("markov:0.0", "markov:0.5", "markov:0.8"),
    seeds=(0, 1, 2, 3, 4), tolerance=1e-2,
    notes="Markov reuse routing; gate scores ~ N(0,1) softmaxed over the K",
)

QWEN3 = LayerConfig(
    name="qwen3", cfg_id=3, E=128, K=8, d=2048, f=768, S=0,
    w_dtype=BF16, x_dtype=BF16, n_values=(1, 2, 3, 4, 5, 6, 7, 8),
    routing=("logits_ar1",), seeds=(0, 1, 2, 3, 4), tolerance=1e-2,
    notes="logits = x . W_r with x_t = 0.7 x_{t-1} + 0.71 N(0,1)",
)

DSV2LITE = LayerConfig(
    name="dsv2lite", cfg_id=4, E=64, K=6, d=2048, f=1408, S=2,
    w_dtype=BF16, x_dtype=BF16, n_values=(1, 2, 3, 4, 5, 6, 7, 8),
    routing=("markov:0.5",), tree_nodes=(16,), seeds=(0, 1, 2, 3, 4),
    tolerance=1e-2,
    notes="2 shared experts always applied; 16-node draft tree (union over all nodes)",
)

DSV3 = LayerConfig(
    name="dsv3", cfg_id=5, E=256, K=8, d=7168, f=2048, S=0,
    w_dtype=FP8, x_dtype=BF16, n_values=(1, 2, 3, 4, 5, 6, 7, 8),
    routing=("iid", "markov:0.5"), tree_nodes=(32,), seeds=(0, 1, 2),
    tolerance=3e-2,
    notes="fp8 e4m3 weights with one fp32 scale per 128x128 block; bf16 activations",
)

ALL = (TINY, OLMOE, QWEN3, DSV2LITE, DSV3)
BY_NAME = {c.name: c for c in ALL}

FP8_BLOCK = 128

