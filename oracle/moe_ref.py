"""Plain, slow CPU reference of the MoE expert operation of a verify pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check of the graft
entry point, and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares
no code with the HIP library (no kernels, headers, helpers or constants);
the two meet only in the seeded input arrays of ``synth``.

Everything is float64 numpy, one definition at a time, in the order and
notation of the pages:

* "Making Every Verified Token Count: Adaptive Verification for MoE
  Speculative Decoding", Sec. 2.2 (MoE verification cost): Eq. (4) router
  top-k of W_g h with normalised selected scores and a weighted sum as the
  layer output; Eq. (5) the union of activated experts over all verified
  tree nodes.
* "Less Experts, Faster Decoding: Cost-Aware Speculative Decoding for MoE",
  Sec. 3, Eq. (1): the verification footprint is the union of the experts
  the verified tokens activate.
* "The Limits of Speculation: Bounding Speculative Decoding in MoE",
  App. A.4.1, Eqs. (A1)-(A2): the same union over a (batch, position)
  micro-batch.
* "Speculative Decoding for Mixture-of-Experts Models: Expert Bytes, Kernel
  Bandwidth and the Best Draft Length", abstract: a deduplicating kernel reads
  each selected expert once per pass, a per-slot kernel once per token;
  Fig. 2 and Table 1: bandwidth on union bytes U*b versus requested bytes
  n*m*b; Table 6: the MLX-LM engine sorts rows by expert before its tiled
  product (the permutation built here).

Readings where the pages are silent (each also listed in the design notes):
ties among equal logits go to the lower expert id; NaN logits rank below
every number; -0.0 and +0.0 compare equal; the selected logits are
normalised by a softmax over the K selected (the pages allow softmax or
sigmoid); the expert FFN is SwiGLU, y = (silu(x W_gate) * (x W_up)) W_down;
shared experts are applied to every token with weight 1 and are read once
per pass by the deduplicating kernel and once per token by the per-slot one.

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

FP8_BLOCK = 128


# ---------------------------------------------------------------- c1: decoding
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE-754 binary32: value = binary32(bits << 16)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_fp8_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP float8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities.

    e == 0           -> (-1)^s * 2^-6 * m/8          (subnormal)
    e == 15, m == 7  -> NaN
    otherwise        -> (-1)^s * 2^(e-7) * (1 + m/8)
    """
    c = np.asarray(codes)
    if c.dtype == np.uint8 and c.size > 256:
        # same formula, evaluated once per code value, then looked up
        return _decode_fp8_formula(np.arange(256))[c]
    return _decode_fp8_formula(c)


def _decode_fp8_formula(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * (2.0 ** -6) * (m / 8.0)
    nor = sign * np.power(2.0, (e - 7).astype(np.float64)) * (1.0 + m / 8.0)
    out = np.where(e == 0, sub, nor)
    out = np.where((e == 15) & (m == 7), np.nan, out)
    return out.astype(np.float64)


def decode_matrix(w: np.ndarray, w_dtype: str, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Stored [rows][cols] matrix -> float64 values (fp8: code value times its block scale)."""
    if w_dtype == "f32":
        return np.asarray(w, dtype=np.float32).astype(np.float64)
    if w_dtype == "bf16":
        return decode_bf16(w)
    if w_dtype == "fp8_e4m3":
        v = decode_fp8_e4m3fn(w)
        rows, cols = v.shape
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        # element (i, j) takes the scale of block (i // 128, j // 128)
        blocks = v.reshape(rows // FP8_BLOCK, FP8_BLOCK, cols // FP8_BLOCK, FP8_BLOCK)
        return (blocks * s[:, None, :, None]).reshape(rows, cols)
    raise ValueError(w_dtype)


def decode_x(x: np.ndarray, x_dtype: str) -> np.ndarray:
    if x_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if x_dtype == "bf16":
        return decode_bf16(x)
    raise ValueError(x_dtype)


class DecodedExpert:
    """The three matrices of one expert in the pages' orientation.

    W_gate, W_up: d x f; W_down: f x d  (stored transposed: one row per output).
    """

    def __init__(self, stored: Dict[str, np.ndarray], w_dtype: str):
        self.W_gate = decode_matrix(stored["w_gate"], w_dtype, stored.get("s_gate")).T
        self.W_up = decode_matrix(stored["w_up"], w_dtype, stored.get("s_up")).T
        self.W_down = decode_matrix(stored["w_down"], w_dtype, stored.get("s_down")).T


def expert_bytes(d: int, f: int, w_dtype: str) -> int:
    """Bytes one expert occupies: three d*f matrices, plus fp8 block scales (fp32)."""
    elem = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[w_dtype]
    b = 3 * d * f * elem
    if w_dtype == "fp8_e4m3":
        b += 3 * (d // FP8_BLOCK) * (f // FP8_BLOCK) * 4
    return b


# ------------------------------------------------------------------ c2: top-K
def _rank_key(value: float, e: int) -> Tuple[int, float, int]:
    # larger logit first; NaN after every number; equal logits: lower id first
    if math.isnan(value):
        return (1, 0.0, e)
    return (0, -value, e)


def route_topk(logits: np.ndarray, K: int) -> Tuple[np.ndarray, np.ndarray]:
    """Eq. (4): indices of the K largest router scores, then softmax over those K.

    Returns ids int32 [n][K] in descending-logit order and gates float64 [n][K].
    """
    lg = np.asarray(logits, dtype=np.float32)
    n, E = lg.shape
    ids = np.empty((n, K), dtype=np.int32)
    gates = np.empty((n, K), dtype=np.float64)
    for t in range(n):
        order = sorted(range(E), key=lambda e: _rank_key(float(lg[t, e]), e))
        sel = order[:K]
        ids[t] = sel
        vals = np.array([float(lg[t, e]) for e in sel], dtype=np.float64)
        top = vals.max()
        ex = np.exp(vals - top)
        gates[t] = ex / ex.sum()
    return ids, gates


# ----------------------------------------------------------------- c3: union
def build_union(ids: np.ndarray, E: int) -> Dict[str, object]:
    """Eq. (1)/(5)/(A2): the distinct experts of all n*K slots, with the slot grouping.

    Slot s = t*K + k.  Outputs (capacity cap = min(n*K, E)):
      U          number of distinct ids (-1 if any id lies outside [0, E))
      union_ids  [cap]    ascending distinct ids, -1 beyond U
      offsets    [cap+1]  offsets[u] = slots routed to union_ids[< u]; n*K beyond U
      perm       [n*K]    slots ordered by (id, slot): the rows sorted by expert
      slot_rank  [n*K]    position of ids[s] in union_ids
    """
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    nk = len(flat)
    cap = min(nk, E)
    if any(v < 0 or v >= E for v in flat):
        return {"U": -1}
    distinct = sorted(set(flat))
    U = len(distinct)
    union_ids = np.full(cap, -1, dtype=np.int32)
    union_ids[:U] = distinct
    position = {e: u for u, e in enumerate(distinct)}
    counts = [0] * U
    for v in flat:
        counts[position[v]] += 1
    offsets = np.full(cap + 1, nk, dtype=np.int32)
    run = 0
    for u in range(U):
        offsets[u] = run
        run += counts[u]
    offsets[U] = run
    perm = np.array(sorted(range(nk), key=lambda s: (flat[s], s)), dtype=np.int32)
    slot_rank = np.array([position[v] for v in flat], dtype=np.int32)
    return {"U": U, "union_ids": union_ids, "offsets": offsets, "perm": perm,
            "slot_rank": slot_rank}


# ------------------------------------------------------------ c4: expert FFN
def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(x_t: np.ndarray, ex: DecodedExpert) -> np.ndarray:
    """One token through one expert: a = x W_gate, v = x W_up, h = silu(a) * v, y = h W_down."""
    a = x_t @ ex.W_gate
    v = x_t @ ex.W_up
    h = silu(a) * v
    return h @ ex.W_down


ExpertSource = Callable[[int], Dict[str, np.ndarray]]


def ffn_perslot(x: np.ndarray, ids: np.ndarray, expert: ExpertSource, shared: ExpertSource,
                S: int, w_dtype: str, x_dtype: str, d: int, f: int):
    """Per-slot mode: the expert of slot (t, k) is read (decoded) once for that slot.

    Shared expert s is read once per token.  Returns y_slots [n][K][d],
    y_shared [n][S][d] and the bytes read.
    """
    xs = decode_x(x, x_dtype)
    n, K = np.asarray(ids).shape
    y = np.zeros((n, K, d))
    ysh = np.zeros((n, S, d))
    read = 0
    eb = expert_bytes(d, f, w_dtype)
    for t in range(n):
        for k in range(K):
            ex = DecodedExpert(expert(int(ids[t, k])), w_dtype)
            read += eb
            y[t, k] = swiglu(xs[t], ex)
        for s in range(S):
            ex = DecodedExpert(shared(s), w_dtype)
            read += eb
            ysh[t, s] = swiglu(xs[t], ex)
    return y, ysh, read


def ffn_dedup(x: np.ndarray, ids: np.ndarray, union: Dict[str, object], expert: ExpertSource,
              shared: ExpertSource, S: int, w_dtype: str, x_dtype: str, d: int, f: int):
    """Deduplicating mode: each union expert is read once and applied to every slot routed to it.

    The per-slot arithmetic is the same call as in ``ffn_perslot``.
    """
    xs = decode_x(x, x_dtype)
    n, K = np.asarray(ids).shape
    y = np.zeros((n, K, d))
    ysh = np.zeros((n, S, d))
    read = 0
    eb = expert_bytes(d, f, w_dtype)
    U = int(union["U"])
    offsets = union["offsets"]
    perm = union["perm"]
    for u in range(U):
        ex = DecodedExpert(expert(int(union["union_ids"][u])), w_dtype)
        read += eb
        for p in range(int(offsets[u]), int(offsets[u + 1])):
            slot = int(perm[p])
            t, k = divmod(slot, K)
            y[t, k] = swiglu(xs[t], ex)
    for s in range(S):
        ex = DecodedExpert(shared(s), w_dtype)
        read += eb
        for t in range(n):
            ysh[t, s] = swiglu(xs[t], ex)
    return y, ysh, read


# ---------------------------------------------------------------- c7: combine
def combine(y_slots: np.ndarray, gates: np.ndarray, y_shared: Optional[np.ndarray]) -> np.ndarray:
    """Layer output: gate-weighted sum over the K slots (k ascending) plus the shared outputs."""
    n, K, d = y_slots.shape
    out = np.zeros((n, d))
    for t in range(n):
        for k in range(K):
            out[t] += float(gates[t, k]) * y_slots[t, k]
        if y_shared is not None:
            for s in range(y_shared.shape[1]):
                out[t] += y_shared[t, s]
    return out


# ------------------------------------------------------------------ c8: bytes
def byte_counts(d: int, f: int, w_dtype: str, K: int, S: int, n: int, U: int) -> Tuple[int, int]:
    """Union bytes (U + S) * b and per-slot requested bytes n * (K + S) * b."""
    b = expert_bytes(d, f, w_dtype)
    return (U + S) * b, n * (K + S) * b


# -------------------------------------------------------- c9: routing statistics
def union_size(ids: np.ndarray) -> int:
    return len(set(int(v) for v in np.asarray(ids).reshape(-1)))


def reuse_last(ids: np.ndarray) -> float:
    """Share of the last token's K experts already chosen by the tokens before it."""
    ids = np.asarray(ids)
    K = ids.shape[1]
    before = set(int(v) for v in ids[:-1].reshape(-1))
    return len(before & set(int(v) for v in ids[-1])) / K


def distinct_share(ids: np.ndarray) -> float:
    """U / (n m): the share of a pass's n*m slots that name distinct experts."""
    ids = np.asarray(ids)
    return union_size(ids) / ids.size


# -------------------------------------------------------------- whole pass
def verify_op(case, mode: str = "dedup") -> Dict[str, object]:
    """Route, union, expert FFN (dedup or per-slot) and combine for one synth case."""
    cfg = case.cfg
    ids, gates = route_topk(case.logits, cfg.K)
    un = build_union(ids, cfg.E)
    if mode == "dedup":
        y, ysh, read = ffn_dedup(case.x, ids, un, case.expert, case.shared, cfg.S,
                                 cfg.w_dtype, cfg.x_dtype, cfg.d, cfg.f)
    else:
        y, ysh, read = ffn_perslot(case.x, ids, case.expert, case.shared, cfg.S,
                                   cfg.w_dtype, cfg.x_dtype, cfg.d, cfg.f)
    out = combine(y, gates, ysh if cfg.S else None)
    ub, rb = byte_counts(cfg.d, cfg.f, cfg.w_dtype, cfg.K, cfg.S, case.n, int(un["U"]))
    return {"ids": ids, "gates": gates, "union": un, "y_slots": y, "y_shared": ysh,
            "out": out, "bytes_read": read, "union_bytes": ub, "requested_bytes": rb}
