"""Host checks of the one-launch pass's unit partition (no GPU).

`moe_unit_partition` runs, on the host, the same range and owner arithmetic
the layer kernel runs on the device (csrc/partition.h): workgroup c streams
units [first[c], first[c+1]) of a phase, and a DOWN group waits for the
workgroups [owner_lo[g], owner_hi[g]] that own its UP units.  A mistake here
on the device would leave a unit unstreamed (zero rows) or let a DOWN group
read H before its owners wrote it, so the properties are pinned against brute
force over every unit:

- the ranges tile the units in order (first[0] = 0, first[G] = ng * upg,
  non-decreasing);
- even split (tile 0): every range holds floor or ceil of ng * upg / G units;
- cost split (tile 8, 16, 32): a unit of a group of cnt tokens costs the
  stated weight (UP: 8 for one tile, 9 per tile beyond; DOWN: 3 + ceil(t/4)
  per tile of t tokens), and workgroup c owns exactly the units whose cost
  prefix P(u) satisfies floor(P(u) * G / total) = c, so every range's cost is
  within one unit of total / G;
- owner_lo / owner_hi are exactly the first and last workgroup whose range
  holds a unit of the group.
"""
from __future__ import annotations

import numpy as np
import pytest

from moe_speculative_decoding_amd import _lib as L


def _owners_brute(first, ng, upg):
    grid = len(first) - 1
    owner = np.empty(ng * upg, dtype=np.int64)
    for c in range(grid):
        owner[first[c]:first[c + 1]] = c
    lo = np.array([owner[g * upg:(g + 1) * upg].min() for g in range(ng)])
    hi = np.array([owner[g * upg:(g + 1) * upg].max() for g in range(ng)])
    return owner, lo, hi


def _cost(cnt, tile, up):
    if up:
        return 8 if cnt <= tile else 9 * -(-cnt // tile)
    w, t = 0, 0
    while t < cnt:
        c = min(tile, cnt - t)
        w += 3 + -(-c // 4)
        t += tile
    return w if w > 0 else 4


CASES = [
    # (ng, upg, grid, tile, up, seed)
    (8, 512, 256, 0, True, 0),        # one token, DeepSeek-V3 UP units
    (57, 1792, 256, 0, False, 1),     # n = 8 DOWN units
    (3, 7, 64, 0, True, 2),           # fewer units than workgroups
    (109, 512, 256, 8, True, 3),      # 32-node tree, fp8 UP tile 8
    (109, 1792, 256, 32, False, 4),   # its DOWN phase
    (159, 512, 256, 8, True, 5),
    (40, 256, 240, 16, True, 6),      # a grid that is not a power of two
    (40, 448, 240, 16, False, 7),
    (5, 3, 37, 8, True, 8),           # tiny ranges, many empty workgroups
    (264, 64, 4096, 32, False, 9),    # the largest table and grid
]


@pytest.mark.parametrize("ng,upg,grid,tile,up,seed", CASES)
def test_partition_tiles_units_and_owners_match_brute_force(ng, upg, grid, tile, up, seed):
    rng = np.random.default_rng(seed)
    counts = rng.integers(1, 6, size=ng)
    if tile:
        # a few groups beyond the tile, as Markov draft trees produce
        big = rng.choice(ng, size=max(1, ng // 20), replace=False)
        counts[big] = rng.integers(tile + 1 if tile < 32 else 17, 33, size=big.size)
    first, lo, hi = L.moe_unit_partition(counts, tile, up, upg, grid)
    nu = ng * upg
    assert first[0] == 0 and first[grid] == nu
    assert np.all(np.diff(first) >= 0)
    owner, blo, bhi = _owners_brute(first, ng, upg)
    assert np.array_equal(lo, blo) and np.array_equal(hi, bhi)
    if tile == 0:
        sizes = np.diff(first)
        assert sizes.min() >= nu // grid and sizes.max() <= -(-nu // grid)
        return
    w = np.array([_cost(int(c), tile, up) for c in counts], dtype=np.int64)
    unit_w = np.repeat(w, upg)
    prefix = np.concatenate([[0], np.cumsum(unit_w)[:-1]])
    total = int(unit_w.sum())
    assert np.array_equal(owner, (prefix * grid) // total)
    per_wg = np.array([unit_w[first[c]:first[c + 1]].sum() for c in range(grid)])
    assert np.all(np.abs(per_wg - total / grid) <= w.max() + 1e-9)


def test_partition_cost_weights_follow_the_stated_rule():
    # two groups of one unit each, [cnt tokens, 1 token], split over as many
    # workgroups as their stated total cost wa + wb: workgroup c then owns
    # the units u with P(u) = c, so the second unit starts at workgroup wa,
    # which pins the first group's weight exactly
    for tile in (8, 16, 32):
        for up in (True, False):
            for cnt in range(1, 33):
                wa, wb = _cost(cnt, tile, up), _cost(1, tile, up)
                first, lo, hi = L.moe_unit_partition([cnt, 1], tile, up, 1, wa + wb)
                assert first[0] == 0 and first[1] == 1, (tile, up, cnt)
                assert list(first[1:wa + 1]) == [1] * wa, (tile, up, cnt, first)
                assert list(first[wa + 1:]) == [2] * wb, (tile, up, cnt, first)
                assert lo.tolist() == [0, wa] and hi.tolist() == [0, wa]


def test_partition_rejects_bad_arguments():
    cnt = np.ones(4, dtype=np.int32)
    out = np.zeros(9, dtype=np.int64)
    lo = np.zeros(4, dtype=np.int32)
    hi = np.zeros(4, dtype=np.int32)
    call = L.lib.moe_unit_partition
    ok = (cnt.ctypes.data, 4, 8, 1, 16, 8, out.ctypes.data, lo.ctypes.data, hi.ctypes.data)
    assert call(*ok) == L.MOE_OK
    assert call(None, *ok[1:]) == L.MOE_ERR_ARG
    assert call(ok[0], 0, *ok[2:]) == L.MOE_ERR_ARG            # no groups
    assert call(ok[0], 4, 12, *ok[3:]) == L.MOE_ERR_ARG        # tile not 0/8/16/32
    assert call(*ok[:4], 0, *ok[5:]) == L.MOE_ERR_ARG          # upg < 1
    assert call(*ok[:5], 5000, *ok[6:]) == L.MOE_ERR_ARG       # grid > 4096
    assert call(*ok[:7], None, ok[8]) == L.MOE_ERR_ARG         # one owner array only
    bad = np.array([1, 40, 1, 1], dtype=np.int32)              # more than 32 tokens
    assert call(bad.ctypes.data, *ok[1:]) == L.MOE_ERR_ARG
