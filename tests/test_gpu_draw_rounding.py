"""The kernels round the draw's hash to fp32 exactly as the oracle does.

The draw is r = fp32(h) * 2^-32 and rounds up when r < p (reading 6 of the design notes' list;
include/gq.h, gq_quantize_pack).  It differs from the unrounded rule h * 2^-32 < p only when
h lies within half a float spacing below p * 2^32, which random inputs almost never hit.
Here each case builds it on purpose: a scale and a value that put p * 2^32 on a chosen float,
and an element counter (through the inverse of the finaliser, tests/draw_helpers.py) whose
hash sits just below that float -- rounding up to it (no round-up under the fp32 rule; the
unrounded rule would round up) or rounding down away from it (round-up under both).  The GPU's
codes, wire lanes and fused means must equal the oracle's bit for bit, on the fast path (every
element below the lowest nonzero level) and on the general path (a neighbour above it makes
the wave take the general path), on both grids, and in the 16-worker bf16 fused pass.
"""
import numpy as np
import pytest
import torch

from tests.draw_helpers import counter_for_hash
from tests.gpu_helpers import dev, first_diff, gq, host, say

pytestmark = pytest.mark.gpu
U, X = 0, 1
SEED = 0x5EED
N = 1024


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def _placed(orc, worker, h):
    """(index_base, i0): the element i0 of a buffer counted from index_base hashes to h."""
    c = counter_for_hash(orc.worker_key(SEED, worker), h)
    i0 = min(c, N // 2)
    base = c - i0
    assert base + N <= 1 << 32
    return base, i0


# (grid, levels, value, p * 2^32, hash, expected level at the element)
CASES = [
    # uniform s = 1, scale 1: u = x = 1/2 + 2^-24 is below the lowest level 1, p * 2^32 = 2^31 + 256
    (U, 1, 0.5 + 2.0 ** -24, (1 << 31) + 256, (1 << 31) + 200, 0),
    (U, 1, 0.5 + 2.0 ** -24, (1 << 31) + 256, (1 << 31) + 100, 1),
    # exponential E = 2 (levels 1/2, 1), u = 1/4 + 2^-25 below 1/2: p = 2u, p * 2^32 = 2^31 + 256
    (X, 2, 0.25 + 2.0 ** -25, (1 << 31) + 256, (1 << 31) + 200, 0),
    (X, 2, 0.25 + 2.0 ** -25, (1 << 31) + 256, (1 << 31) + 100, 1),
    # exponential E = 2, u = 3/4 + 2^-24 above 1/2: p = 2u - 1, p * 2^32 = 2^31 + 512
    (X, 2, 0.75 + 2.0 ** -24, (1 << 31) + 512, (1 << 31) + 400, 1),
    (X, 2, 0.75 + 2.0 ** -24, (1 << 31) + 512, (1 << 31) + 300, 2),
]


@pytest.mark.parametrize("general", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_quantize_pack_and_wire_round_the_draw(orc, case, general):
    grid, levels, x, thr, h, want = CASES[case]
    assert np.float32(x) == x and float(np.float32(thr)) == thr
    base, i0 = _placed(orc, 0, h)
    xs = np.full(N, np.float32(x), np.float32)
    if general:
        xs[i0 ^ 1] = np.float32(1.5 if grid == U else 0.6)  # at or above the lowest nonzero level
    S = np.ones(1, np.float32)
    ref = orc.quantize(xs, S, grid, levels, SEED, 0, base)
    assert ref[i0] == want, (ref[i0], want)
    say("draw rounding quantize_pack", grid, levels, hex(h), general)
    g = gq()
    bits = 8
    codes = g.quantize_pack(dev(xs), dev(S), grid, levels, bits, SEED, 0, base)
    exp_codes = orc.pack(ref, grid, bits)
    assert np.array_equal(host(codes), exp_codes), first_diff(host(codes), exp_codes)
    world = 2
    pay = g.quantize_wire(dev(xs), dev(S), grid, levels, SEED, 0, world, index_base=base)
    exp_pay = orc.wire_encode(ref, grid, levels, world)
    assert np.array_equal(host(pay), exp_pay), first_diff(host(pay), exp_pay)


@pytest.mark.parametrize("h,want", [((1 << 31) + (1 << 24) - 100, 0),
                                    ((1 << 31) + (1 << 24) - 200, 1)])
def test_bf16_fused_pass_rounds_the_draw(orc, h, want):
    """16 bf16 workers (the double-buffered pass, whose fast path scales |x| by inv * 2^32 in
    one product): s = 7, scale 7, x = 1/2 + 2^-8 (a bf16 value), so p * 2^32 = 2^31 + 2^24 on
    the fast path; worker 0's hash at element i0 is placed just below it."""
    K, levels = 16, 7
    base, i0 = _placed(orc, 0, h)
    x = np.float32(0.5 + 2.0 ** -8)
    xb = (np.full(N, x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    xs = [xb.copy() for _ in range(K)]
    S = np.full(1, 7.0, np.float32)
    q0 = orc.quantize(xs[0], S, U, levels, SEED, 0, base)
    assert q0[i0] == want, (q0[i0], want)
    qs = [orc.pack(orc.quantize(xs[k], S, U, levels, SEED, k, base), U, 4) for k in range(K)]
    sums, over = orc.accumulate(qs, N, U, 4, 16)
    assert over == 0
    ref = orc.dequantize(sums, S, U, levels, K, out_dtype=1)
    say("draw rounding bf16 fused", hex(h))
    g = gq()
    out = g.fused_mean([dev(a) for a in xs], dev(S), U, levels, 4, SEED, 16, 1, index_base=base)
    assert np.array_equal(host(out), ref), first_diff(host(out), ref)
