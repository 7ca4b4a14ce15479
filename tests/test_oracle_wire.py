"""Pins of the oracle's summable wire payload (CPU only).

Reading of "the codes of all workers can be summed by Allreduce" for a collective that sums
unsigned 32-bit words (RCCL has no 16-bit integer sum): each element travels as the unsigned
lane lin + o, o = s (uniform) or 2^(E-1) (exponential), in the smallest of 1, 2 or 4 bytes
whose range holds world * 2o.  Pinned here: the width rule, the byte layout (hand-worked
fixtures), that summing world payloads word by word never carries between lanes, and that
the decoded sums are exactly the integer sums of the code path, so the mean decoded from the
wire equals the allreduce mean bit for bit.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "wire_layout.json")
U, X = 0, 1


def _offset(grid, levels):
    return 2 ** (levels - 1) if grid == X else levels


@pytest.mark.parametrize("grid", [U, X])
def test_lane_width_is_the_smallest_that_holds_the_sum(orc, grid):
    for levels in (range(1, 128) if grid == U else range(1, 20)):
        for world in (1, 2, 3, 4, 8, 16, 64, 255, 1000):
            w = orc.wire_lane_bytes(grid, levels, world)
            top = world * 2 * _offset(grid, levels)
            if top > 2 ** 32 - 1:
                assert w == 0
                continue
            assert w in (1, 2, 4)
            assert top <= 2 ** (8 * w) - 1
            if w > 1:
                assert top > 2 ** (8 * (w // 2)) - 1


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"])
def test_wire_layout_golden(orc, case):
    grid = U if case["grid"] == "uniform" else X
    assert orc.wire_lane_bytes(grid, case["levels"], case["world"]) == case["lane_bytes"]
    got = orc.wire_encode(np.array(case["q"], np.int32), grid, case["levels"], case["world"])
    assert got.tolist() == case["bytes"]


@pytest.mark.parametrize("grid,levels,world,bits", [(U, 127, 8, 8), (U, 7, 16, 4),
                                                    (X, 7, 8, 4), (U, 31, 4, 8), (U, 1, 127, 4),
                                                    (X, 8, 64, 8)])
def test_word_sums_never_carry_and_decode_to_the_integer_sums(orc, grid, levels, world, bits):
    rng = np.random.default_rng(levels * 100 + world)
    n = 1003
    lo, hi = -levels, levels
    qs = []
    for k in range(world):
        q = rng.integers(lo, hi + 1, n).astype(np.int32)
        q[:8] = hi if k % 2 == 0 else hi   # every worker at the top level
        q[8:16] = lo                       # every worker at the bottom level
        qs.append(q)
    payload = orc.wire_sum([orc.wire_encode(q, grid, levels, world) for q in qs])
    sums = orc.wire_decode(payload, n, grid, levels, world)
    ref, over = orc.accumulate([orc.pack(q, grid, bits) for q in qs], n, grid, bits, 32)
    assert over == 0
    assert np.array_equal(sums, ref)
    top = world * _offset(grid, levels)
    assert (sums[:8] == top).all() and (sums[8:16] == -top).all()


@pytest.mark.parametrize("grid,levels,bits", [(U, 127, 8), (X, 7, 4)])
def test_mean_from_the_wire_equals_the_allreduce_mean(orc, grid, levels, bits):
    rng = np.random.default_rng(3 + grid)
    K, n = 5, 4099
    off = [0, 1024, 1032, n]
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(K)]
    res = orc.allreduce_mean(xs, grid, levels, bits, 32, 7, 0, off)
    payload = orc.wire_sum([orc.wire_encode(q, grid, levels, K) for q in res["levels"]])
    sums = orc.wire_decode(payload, n, grid, levels, K)
    assert np.array_equal(sums, res["sums"])
    mean = orc.dequantize(sums, res["scale"], grid, levels, K, offsets=off)
    assert np.array_equal(mean, res["mean"])
