"""Seeded synthetic inputs for the MoE verify-pass expert operation.

Both the oracle and the GPU path consume these arrays; this module performs
none of the method's arithmetic (no top-K, union, FFN, combine or byte
accounting).  It only draws random numbers, rounds them to the storage
formats with library conversions (torch's round-to-nearest-even casts to
bfloat16 and float8_e4m3fn), and places them in the memory layout the
library's C ABI documents:

* tokens ``x``                 [n][d]   (f32, or bf16 stored as uint16 bits)
* router logits                [n][E]   f32
* ``w_gate``, ``w_up``         [E][f][d]  (output-major: one row per output j)
* ``w_down``                   [E][d][f]
* fp8 block scales (DeepSeek-V3 shape) ``s_gate``/``s_up`` [E][f/128][d/128],
  ``s_down`` [E][d/128][f/128]; stored value = decode(code) * scale.

Recipes (the pages give shapes and routing statistics, not values):

* x ~ N(0, 1) per element; for the Qwen3 shape the tokens follow
  x_t = 0.7 x_{t-1} + 0.71 e_t with e_t ~ N(0, 1) (consecutive-token
  correlation of a real text stream).
* every expert matrix ~ N(0, 1/d); router W_r [d][E] ~ N(0, 1/d).
* fp8: per 128x128 block, scale = amax / 448 (amax = 0 gives 1), codes =
  round-to-nearest-even of w / scale clipped to [-448, 448].
* Markov routing: token 0 (or the tree root) draws K distinct experts
  uniformly; every later token keeps each of its predecessor's experts with
  probability p and fills up to K without replacement, uniformly, from the
  E - K experts the predecessor did not select.  In a draft tree the
  predecessor is the parent, parent(i) = (i - 1) // 2.
* iid routing: K distinct experts uniformly, independently per token.
* Realised logits for generated routing: the selected experts get logits
  ~ N(0, 1) (the gate scores), every other expert gets a logit strictly
  below the token's smallest selected logit, so the top-K of the logits is
  exactly the generated set.

Random streams: numpy ``default_rng([seed, cfg_id, layer, window, stream])``
for per-window arrays and ``default_rng([seed, cfg_id, layer, 0xE0000 + e])``
for expert e's weights (shared expert s uses e = E + s).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from .configs import BF16, F32, FP8, FP8_BLOCK, LayerConfig

STREAM_X = 0
STREAM_WR = 1
STREAM_ROUTE = 2
STREAM_SCORES = 3
STREAM_FILL = 4
EXPERT_STREAM_BASE = 0xE0000

FP8_MAX = 448.0


def window_rng(cfg: LayerConfig, seed: int, layer: int, window: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, cfg.cfg_id, layer, window, stream])


def expert_rng(cfg: LayerConfig, seed: int, layer: int, e: int) -> np.random.Generator:
    return np.random.default_rng([seed, cfg.cfg_id, layer, EXPERT_STREAM_BASE + e])


# ----------------------------------------------------------------- storage casts
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even (torch)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_fp8_codes(a: np.ndarray) -> np.ndarray:
    """float32 values already within [-448, 448] -> e4m3fn codes (uint8), RNE (torch)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def quantize_fp8_blocks(w: np.ndarray):
    """[rows][cols] float32 -> (codes uint8 [rows][cols], scales f32 [rows/128][cols/128]).

    float32 throughout (torch CPU ops): scale = amax / 448, codes = RNE of the
    clipped quotient."""
    rows, cols = w.shape
    rb, cb = rows // FP8_BLOCK, cols // FP8_BLOCK
    blocks = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).view(
        rb, FP8_BLOCK, cb, FP8_BLOCK)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blocks / scale[:, None, :, None]).clamp_(-FP8_MAX, FP8_MAX).reshape(rows, cols)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale.numpy().astype(np.float32)


def store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return to_bf16_bits(a)
    raise ValueError(dtype)


# ----------------------------------------------------------------------- weights
def expert_weights(cfg: LayerConfig, e: int, seed: int = 0, layer: int = 0) -> Dict[str, np.ndarray]:
    """Weights of expert e (routed e < E, shared e = E + s) in storage layout.

    Normals come from torch's CPU generator seeded from the expert's numpy
    seed sequence (faster than numpy for the 44M values of a DeepSeek-V3
    expert)."""
    g = torch.Generator().manual_seed(int(expert_rng(cfg, seed, layer, e).integers(0, 2 ** 62)))
    std = 1.0 / float(np.sqrt(cfg.d))

    def draw(shape):
        return (torch.randn(shape, generator=g, dtype=torch.float32) * std).numpy()

    wg = draw((cfg.f, cfg.d))
    wu = draw((cfg.f, cfg.d))
    wd = draw((cfg.d, cfg.f))
    if cfg.w_dtype == FP8:
        qg, sg = quantize_fp8_blocks(wg)
        qu, su = quantize_fp8_blocks(wu)
        qd, sd = quantize_fp8_blocks(wd)
        return {"w_gate": qg, "w_up": qu, "w_down": qd, "s_gate": sg, "s_up": su, "s_down": sd}
    return {"w_gate": store(wg, cfg.w_dtype), "w_up": store(wu, cfg.w_dtype),
            "w_down": store(wd, cfg.w_dtype)}


def stack_experts(cfg: LayerConfig, experts: Sequence[int], count: int, seed: int = 0,
                  layer: int = 0, base: int = 0) -> Dict[str, np.ndarray]:
    """[count][...] arrays; slot i holds expert base + i if listed in ``experts``, else zeros."""
    want = set(int(e) for e in experts)
    out: Dict[str, np.ndarray] = {}
    for i in range(count):
        if base + i not in want:
            continue
        w = expert_weights(cfg, base + i, seed, layer)
        for k, v in w.items():
            if k not in out:
                out[k] = np.zeros((count,) + v.shape, dtype=v.dtype)
            out[k][i] = v
    if not out:  # nothing requested: still return correctly shaped zero arrays
        w = expert_weights(cfg, base, seed, layer)
        out = {k: np.zeros((count,) + v.shape, dtype=v.dtype) for k, v in w.items()}
    return out


# ----------------------------------------------------------------------- routing
def tree_parents(nodes: int) -> np.ndarray:
    """Heap-shaped draft tree: parent(i) = (i - 1) // 2, root has parent -1."""
    p = np.arange(nodes) - 1
    p[1:] = (np.arange(1, nodes) - 1) // 2
    p[0] = -1
    return p


def chain_parents(n: int) -> np.ndarray:
    p = np.arange(n) - 1
    return p


def markov_sets(g: np.random.Generator, parents: np.ndarray, E: int, K: int, p: float) -> np.ndarray:
    n = len(parents)
    ids = np.empty((n, K), dtype=np.int32)
    for t in range(n):
        if parents[t] < 0:
            ids[t] = g.choice(E, K, replace=False)
            continue
        prev = ids[parents[t]]
        keep = prev[g.random(K) < p]
        pool = np.setdiff1d(np.arange(E), prev)
        fill = g.choice(pool, K - len(keep), replace=False)
        ids[t] = np.concatenate([keep, fill])
    return ids


def iid_sets(g: np.random.Generator, n: int, E: int, K: int) -> np.ndarray:
    return np.stack([g.choice(E, K, replace=False) for _ in range(n)]).astype(np.int32)


def realise_logits(g_scores: np.random.Generator, g_fill: np.random.Generator,
                   sets: np.ndarray, E: int) -> np.ndarray:
    n, K = sets.shape
    logits = np.empty((n, E), dtype=np.float32)
    for t in range(n):
        scores = g_scores.standard_normal(K).astype(np.float32)
        floor = scores.min() - np.float32(1.0)
        logits[t] = floor - g_fill.random(E).astype(np.float32)
        logits[t, sets[t]] = scores
    return logits


# ------------------------------------------------------------------------ a case
@dataclass
class Case:
    cfg: LayerConfig
    n: int
    routing: str
    seed: int
    layer: int
    window: int
    x: np.ndarray                 # [n][d] storage dtype (float32 or uint16 bf16 bits)
    logits: np.ndarray            # [n][E] float32
    parents: np.ndarray           # [n] predecessor index (-1: none)
    gen_sets: Optional[np.ndarray] = None   # generated routing sets, if any
    _experts: Dict[int, Dict[str, np.ndarray]] = field(default_factory=dict, repr=False)

    def expert(self, e: int) -> Dict[str, np.ndarray]:
        if e not in self._experts:
            self._experts[e] = expert_weights(self.cfg, e, self.seed, self.layer)
        return self._experts[e]

    def shared(self, s: int) -> Dict[str, np.ndarray]:
        return self.expert(self.cfg.E + s)


def make_case(cfg: LayerConfig, n: int, routing: Optional[str] = None, seed: int = 0,
              window: int = 0, layer: int = 0, tree: bool = False) -> Case:
    routing = routing or cfg.routing[0]
    parents = tree_parents(n) if tree else chain_parents(n)
    gx = window_rng(cfg, seed, layer, window, STREAM_X)
    gen_sets = None
    if routing == "logits_ar1":
        xs = np.empty((n, cfg.d), dtype=np.float64)
        for t in range(n):
            eps = gx.standard_normal(cfg.d)
            xs[t] = eps if parents[t] < 0 else 0.7 * xs[parents[t]] + 0.71 * eps
        x = store(xs.astype(np.float32), cfg.x_dtype)
    else:
        x = store(gx.standard_normal((n, cfg.d), dtype=np.float32), cfg.x_dtype)

    if routing.startswith("logits"):
        gw = window_rng(cfg, seed, layer, 0, STREAM_WR)   # one router per layer
        wr = (gw.standard_normal((cfg.d, cfg.E)) / np.sqrt(cfg.d)).astype(np.float32)
        xv = x.astype(np.float64) if cfg.x_dtype == F32 else \
            torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
        logits = (xv @ wr.astype(np.float64)).astype(np.float32)
    else:
        gr = window_rng(cfg, seed, layer, window, STREAM_ROUTE)
        if routing == "iid":
            gen_sets = iid_sets(gr, n, cfg.E, cfg.K)
        elif routing.startswith("markov:"):
            p = float(routing.split(":", 1)[1])
            gen_sets = markov_sets(gr, parents, cfg.E, cfg.K, p)
        else:
            raise ValueError(routing)
        logits = realise_logits(window_rng(cfg, seed, layer, window, STREAM_SCORES),
                                window_rng(cfg, seed, layer, window, STREAM_FILL),
                                gen_sets, cfg.E)
    return Case(cfg=cfg, n=n, routing=routing, seed=seed, layer=layer, window=window,
                x=x, logits=logits, parents=parents, gen_sets=gen_sets)


# ------------------------------------------------- device-resident layer weights
def device_layer_weights(cfg: LayerConfig, seed: int, layer: int, device, count: Optional[int] = None,
                         shared: bool = False) -> Dict[str, "torch.Tensor"]:
    """Weights of a whole layer drawn directly on the device (large benchmark layers).

    Same recipe as ``expert_weights`` (N(0, 1/d) per element; fp8 codes with one
    scale per 128x128 block), drawn from torch's device generator seeded with
    (seed, cfg_id, layer, shared); the values therefore differ from the host
    generator's, and a check against the oracle copies the experts it needs back.
    """
    count = count if count is not None else (cfg.S if shared else cfg.E)
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1000003 + cfg.cfg_id) * 10007 + layer) * 2 + int(shared))
    std = 1.0 / float(np.sqrt(cfg.d))
    out: Dict[str, torch.Tensor] = {}
    shapes = {"w_gate": (cfg.f, cfg.d), "w_up": (cfg.f, cfg.d), "w_down": (cfg.d, cfg.f)}
    for name, (r, c) in shapes.items():
        w = torch.randn((count, r, c), generator=g, device=device, dtype=torch.float32)
        w.mul_(std)
        if cfg.w_dtype == FP8:
            blocks = w.view(count, r // FP8_BLOCK, FP8_BLOCK, c // FP8_BLOCK, FP8_BLOCK)
            amax = blocks.abs().amax(dim=(2, 4))
            scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
            blocks.div_(scale[:, :, None, :, None]).clamp_(-FP8_MAX, FP8_MAX)
            out[name] = w.to(torch.float8_e4m3fn).view(torch.uint8)
            out["s" + name[1:]] = scale.contiguous()
        elif cfg.w_dtype == BF16:
            out[name] = w.to(torch.bfloat16).view(torch.int16)
        else:
            out[name] = w
        del w
    return out


# ---------------------------------------------------------- draft trees
def draft_tree(nodes: int, seed: int, width: int = 8, fanout: int = 4,
               p_one: float = 0.0):
    """A draft tree of `nodes` nodes in breadth-first order (parent(v) < v;
    -1 = a child of the root token), built level by level with at most
    `width` nodes per level and `fanout` children per node, plus each node's
    draft probability given its parent: the children of one node share a
    random split of at most probability 1 (the rest stays with tokens not
    drafted).  With p_one > 0 that share of edges gets probability exactly 1
    (equal scores of parent and child).  Returns (parent int32, q float32)."""
    g = np.random.default_rng([seed, 7001, nodes])
    parent = []
    prev = [-1]
    while len(parent) < nodes:
        level = []
        slots = [p for p in prev for _ in range(fanout if p >= 0 else width)]
        g.shuffle(slots)
        for p in sorted(slots[:min(width, nodes - len(parent))]):
            level.append(len(parent))
            parent.append(p)
        prev = level
    parent = np.asarray(parent, dtype=np.int32)
    q = np.zeros(nodes, dtype=np.float32)
    for p in np.unique(parent):
        kids = np.flatnonzero(parent == p)
        share = g.dirichlet(np.ones(len(kids) + 1))[:len(kids)]
        q[kids] = np.sort(share)[::-1].astype(np.float32)
    if p_one > 0:
        q[g.random(nodes) < p_one] = 1.0
    return parent, q


def step_costs(k_max: int, seed: int):
    """An increasing cost table C(1..k_max) (profiled step latency, arbitrary
    unit): a fixed part plus a concave rise, with small noise."""
    g = np.random.default_rng([seed, 7002, k_max])
    k = np.arange(1, k_max + 1, dtype=np.float64)
    c = 10.0 + 1.5 * k ** 0.8 + g.uniform(0.0, 0.05, k_max)
    return np.maximum.accumulate(c).astype(np.float32)


def expert_bitsets(sets, layers: int, experts: int) -> np.ndarray:
    """(layer, expert) sets -> uint64 [len(sets)][W]: bit l*experts + e in word
    (l*experts + e) // 64 (the layout of the selection kernels' footprints)."""
    bits = layers * experts
    W = (bits + 63) // 64
    out = np.zeros((len(sets), W), dtype=np.uint64)
    for i, s in enumerate(sets):
        for (l, e) in s:
            b = l * experts + e
            out[i, b // 64] |= np.uint64(1) << np.uint64(b % 64)
    return out


def predicted_sets(nodes: int, layers: int, experts: int, k: int, seed: int, parent=None,
                   p_keep: float = 0.6):
    """Predicted (layer, expert) sets of draft nodes: per layer k experts; a
    node keeps each of its parent's experts with probability p_keep and fills
    the rest uniformly (Markov reuse along tree edges, as the routing recipe)."""
    g = np.random.default_rng([seed, 7003, nodes, layers, experts])
    out = []
    for v in range(nodes):
        p = -1 if parent is None else int(parent[v])
        s = set()
        for l in range(layers):
            prev = sorted(e for (ll, e) in out[p] if ll == l) if p >= 0 else []
            keep = [e for e in prev if g.random() < p_keep]
            rest = [e for e in range(experts) if e not in keep]
            fill = g.choice(rest, size=k - len(keep), replace=False).tolist() if k > len(keep) else []
            s.update((l, int(e)) for e in keep + fill)
        out.append(s)
    return out


def reference_sequence_inputs(N: int, L: int, seed: int, E: int = 128, K: int = 8):
    """Inputs of the draft-length oracle over a reference sequence of N tokens:
    q [N] float64, the draft model's probability of each reference token given
    its prefix (runs of easy and hard text: Beta draws whose parameters switch
    every 8-40 tokens), and cost [N][L][L+1] float64 in ms, Cost(i, k, a) of a
    step at position i with k drafts of which a are accepted: a draft part
    linear in k plus a target part linear in the unique experts the k+1
    positions activate (independent routing of E experts, K per token, more
    for the rejected tail) and in the prefix length.  Coefficients are
    arbitrary, of the order of a 30B-parameter MoE on one GPU."""
    g = np.random.default_rng([seed, 7004, N, L])
    q = np.empty(N)
    i = 0
    while i < N:
        run = int(g.integers(8, 41))
        a, b = (8.0, 1.5) if g.random() < 0.5 else (1.5, 2.5)
        q[i:i + run] = g.beta(a, b, size=min(run, N - i))
        i += run
    k = np.arange(1, L + 1, dtype=np.float64)[None, :, None]
    a = np.arange(L + 1, dtype=np.float64)[None, None, :]
    pos = np.arange(N, dtype=np.float64)[:, None, None]
    u_mean = E * (1.0 - (1.0 - K / E) ** (k + 1))
    junk = np.maximum(k - a, 0.0)
    U = u_mean * (1.0 + 0.05 * g.standard_normal((N, L, L + 1))) + 0.5 * junk
    cost = (0.459 * k + 0.073) + 11.0 + 0.06 * U + 2e-4 * (512 + pos)
    return q, cost
