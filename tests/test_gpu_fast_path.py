"""The fused pass's fast path must give the general path's results bit for bit.

A worker's batch in which every |x| lies below the smallest value whose scaled magnitude
reaches the lowest nonzero level (2^(1-E) on the exponential grid; 1 on the uniform grid, where
the 16-worker bf16 pass uses the shortcut) is quantised without the clamp, floor and level
selection.  These inputs are built around that threshold, computed here in numpy's fp32
arithmetic from the scale the kernel is given: batches of small values, some holding the
largest representable value below the threshold (the fast path at its edge), some holding the
threshold itself or the next value above it in one worker and one lane (that batch falls back
to the general path while the other workers' batches stay fast).  Sums and means are compared
with the oracle bit for bit, for fp32 and bf16 elements, both grids and several worker counts.
"""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import dev, first_diff, gq, host, say

pytestmark = pytest.mark.gpu
U, X = 0, 1


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def _threshold(inv, bound):
    """Smallest fp32 a with fl(a * inv) >= bound (numpy fp32 products round to nearest even)."""
    inv, bound = np.float32(inv), np.float32(bound)
    a = np.float32(bound / inv)
    while a > 0 and np.float32(np.nextafter(a, np.float32(0)) * inv) >= bound:
        a = np.nextafter(a, np.float32(0))
    while np.float32(a * inv) < bound:
        a = np.nextafter(a, np.float32(np.inf))
    return np.float32(a)


def _bf16_below_at(a):
    """Largest bf16 value below a and smallest bf16 value at or above a (as fp32)."""
    bits = np.array([a], np.float32).view(np.uint32)[0]
    lo = np.array([bits & 0xFFFF0000], np.uint32).view(np.float32)[0]
    if lo >= a:
        lo = np.array([(bits & 0xFFFF0000) - 0x10000], np.uint32).view(np.float32)[0]
    hi = np.array([(np.array([lo], np.float32).view(np.uint32)[0]) + 0x10000],
                  np.uint32).view(np.float32)[0]
    assert lo < a <= hi
    return np.float32(lo), np.float32(hi)


def _to_bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


CASES = [(g, lv, b, K, dt) for (g, lv, b) in [(U, 7, 4), (U, 127, 8), (X, 7, 4)]
         for K in (1, 3, 8, 16) for dt in ("f32", "bf16")]


@pytest.mark.parametrize("grid,levels,bits,K,dt", CASES)
def test_fast_path_matches_general_path(orc, grid, levels, bits, K, dt):
    say("fast path", grid, levels, bits, K, dt)
    g = gq()
    rng = np.random.default_rng(1000 * grid + 10 * K + levels + (dt == "bf16"))
    n = 2 * 8192 + 1000 + 5
    S = np.float32(1.7)
    if grid == U:
        inv, bound = np.float32(np.float32(levels) / S), np.float32(1.0)
    else:
        inv, bound = np.float32(np.float32(1.0) / S), np.float32(2.0 ** (1 - levels))
    thr = _threshold(inv, bound)
    if dt == "bf16":
        below, at = _bf16_below_at(thr)
    else:
        below, at = np.nextafter(thr, np.float32(0)), thr
    above = np.nextafter(at, np.float32(np.inf)) if dt == "f32" else np.array(
        [np.array([at], np.float32).view(np.uint32)[0] + 0x10000], np.uint32).view(np.float32)[0]
    assert np.float32(below * inv) < bound <= np.float32(at * inv)
    xs = []
    for k in range(K):
        x = (rng.standard_normal(n) * float(thr) * 0.05).astype(np.float32)
        x[rng.random(n) < 0.02] = 0.0
        # the edge of the fast path: the largest value below the threshold, either sign
        for i in rng.choice(n, 40, replace=False):
            x[i] = below if rng.random() < 0.5 else -below
        # one worker, one lane: the threshold itself or the value above it
        if k == K // 2:
            for i in rng.choice(n, 12, replace=False):
                x[i] = rng.choice([at, above, -at, -above])
        if dt == "bf16":
            x = _to_bf16_bits(x)
        xs.append(x)
    acc_bits = 16 if K * (levels if grid == U else 1 << (levels - 1)) < (1 << 15) else 32
    ref = orc.allreduce_mean(xs, grid, levels, bits, acc_bits, 77, 0, scale=[S])
    xd = [dev(x) for x in xs]
    Sd = dev(np.array([S], np.float32))
    mean = g.fused_mean(xd, Sd, grid, levels, bits, 77, acc_bits)
    assert np.array_equal(host(mean), ref["mean"]), first_diff(host(mean), ref["mean"])
    sd = torch.empty(n, dtype=torch.int16 if acc_bits == 16 else torch.int32, device="cuda")
    mean2 = g.fused_mean(xd, Sd, grid, levels, bits, 77, acc_bits, sums=sd)
    assert np.array_equal(host(sd), ref["sums"]), first_diff(host(sd), ref["sums"])
    assert np.array_equal(host(mean2), ref["mean"])
    # the planted values reach the levels they should: some sums are nonzero
    assert np.any(ref["sums"] != 0)


@pytest.mark.parametrize("K,dt", [(1, "f32"), (3, "f32"), (8, "f32"), (16, "bf16"), (5, "bf16")])
@pytest.mark.parametrize("grid,levels", [(X, 7), (U, 7)])
def test_worker_mean_fast_path(orc, grid, levels, K, dt):
    """The per-worker-scale mean (QSGD / NUQSGD) at each worker's own lowest level: values just
    below, at and above the threshold derived from that worker's scale, bit-exact means.  (The
    fused pass's shortcut measured slower in this kernel and is not used there; these inputs
    keep the level boundary under test for the baselines too.)"""
    say("worker mean fast path", grid, levels, K, dt)
    g = gq()
    rng = np.random.default_rng(5000 + 10 * K + grid + (dt == "bf16"))
    n = 2 * 8192 + 777
    off = np.array([0, 8192, n], np.int64)
    Sw = np.array([[np.float32(1.3 * (1.5 ** k) * (1 + 0.37 * s)) for s in range(2)]
                   for k in range(K)], np.float32)
    xs = []
    for k in range(K):
        x = np.empty(n, np.float32)
        for s in range(2):
            S = Sw[k, s]
            if grid == U:
                inv, bound = np.float32(np.float32(levels) / S), np.float32(1.0)
            else:
                inv, bound = np.float32(np.float32(1.0) / S), np.float32(2.0 ** (1 - levels))
            thr = _threshold(inv, bound)
            if dt == "bf16":
                below, at = _bf16_below_at(thr)
                above = np.array([np.array([at], np.float32).view(np.uint32)[0] + 0x10000],
                                 np.uint32).view(np.float32)[0]
            else:
                below, at = np.nextafter(thr, np.float32(0)), thr
                above = np.nextafter(at, np.float32(np.inf))
            lo, hi = off[s], off[s + 1]
            seg = (rng.standard_normal(hi - lo) * float(thr) * 0.05).astype(np.float32)
            for i in rng.choice(hi - lo, 30, replace=False):
                seg[i] = below if rng.random() < 0.5 else -below
            if k == K // 2:
                for i in rng.choice(hi - lo, 6, replace=False):
                    seg[i] = rng.choice([at, above, -at, -above])
            x[lo:hi] = seg
        xs.append(_to_bf16_bits(x) if dt == "bf16" else x)
    ref = orc.worker_mean(xs, Sw, grid, levels, 31, 0, off, 0)
    got = g.worker_mean([dev(x) for x in xs], dev(np.ascontiguousarray(Sw)), grid, levels, 31,
                        0, 0, off)
    assert np.array_equal(host(got), ref), first_diff(host(got), ref)


@pytest.mark.parametrize("grid,levels,world,dt", [(U, 7, 16, "bf16"), (U, 127, 8, "f32"),
                                                  (X, 7, 8, "f32"), (X, 7, 16, "bf16")])
def test_wire_quantiser_fast_path(orc, grid, levels, world, dt):
    """The wire payload's quantiser takes the same shortcut per part: payload bytes around the
    threshold equal the oracle's encoding of its own levels."""
    say("wire fast path", grid, levels, world, dt)
    g = gq()
    rng = np.random.default_rng(7000 + 10 * world + grid + levels)
    n = 2 * 8192 + 999
    S = np.float32(2.3)
    if grid == U:
        inv, bound = np.float32(np.float32(levels) / S), np.float32(1.0)
    else:
        inv, bound = np.float32(np.float32(1.0) / S), np.float32(2.0 ** (1 - levels))
    thr = _threshold(inv, bound)
    if dt == "bf16":
        below, at = _bf16_below_at(thr)
        above = np.array([np.array([at], np.float32).view(np.uint32)[0] + 0x10000],
                         np.uint32).view(np.float32)[0]
    else:
        below, at = np.nextafter(thr, np.float32(0)), thr
        above = np.nextafter(at, np.float32(np.inf))
    x = (rng.standard_normal(n) * float(thr) * 0.05).astype(np.float32)
    for i in rng.choice(n, 60, replace=False):
        x[i] = below if rng.random() < 0.5 else -below
    for i in rng.choice(n, 10, replace=False):
        x[i] = rng.choice([at, above, -at, -above])
    if dt == "bf16":
        x = _to_bf16_bits(x)
    q = orc.quantize(x, [S], grid, levels, 5, 3)
    ref = orc.wire_encode(q, grid, levels, world)
    got = g.quantize_wire(dev(x), dev(np.array([S], np.float32)), grid, levels, 5, 3, world)
    assert np.array_equal(host(got), ref), first_diff(host(got), ref)



# NaN (quiet and signalling patterns, either sign) and infinities; the NaN patterns keep their
# mantissa bits in the upper half, so they stay NaN as bf16
NONFINITE = np.array([0x7FC00000, 0xFFC00000, 0x7F810000, 0xFF810000, 0x7F800000, 0xFF800000],
                     np.uint32).view(np.float32)


@pytest.mark.parametrize("grid,levels,bits,K,dt", [(U, 7, 4, 16, "bf16"), (X, 7, 4, 16, "bf16"),
                                                   (X, 7, 4, 8, "f32"), (X, 7, 4, 3, "f32")])
def test_nonfinite_element_in_a_small_batch(orc, grid, levels, bits, K, dt):
    """Under a caller-given finite scale, a NaN or an infinity among values that all lie below
    the threshold: the lane's largest magnitude must fail the threshold, so that its batch takes
    the general path, which clamps the element to the top level as the oracle does; every other
    batch stays on the fast path.  Sums and means bit-exact with the oracle."""
    say("fast path non-finite", grid, levels, bits, K, dt)
    g = gq()
    rng = np.random.default_rng(9000 + 10 * K + grid)
    n = 3 * 8192 + 77
    S = np.float32(1.9)
    inv = np.float32(np.float32(levels) / S) if grid == U else np.float32(np.float32(1.0) / S)
    bound = np.float32(1.0) if grid == U else np.float32(2.0 ** (1 - levels))
    thr = _threshold(inv, bound)
    xs, xs0, planted = [], [], []
    for k in range(K):
        x = (rng.standard_normal(n) * float(thr) * 0.05).astype(np.float32)
        x0 = x.copy()
        if k % 2 == 1:  # three non-finite values in every other worker, in different chunks
            for t, i in enumerate(rng.choice(n, 3, replace=False)):
                x[i] = NONFINITE[(k + t) % len(NONFINITE)]
                x0[i] = 0.0
                planted.append(i)
        xs.append(_to_bf16_bits(x) if dt == "bf16" else x)
        xs0.append(_to_bf16_bits(x0) if dt == "bf16" else x0)
    acc_bits = 16 if K * (levels if grid == U else 1 << (levels - 1)) < (1 << 15) else 32
    ref = orc.allreduce_mean(xs, grid, levels, bits, acc_bits, 91, 0, scale=[S])
    # each planted element takes the top level: its sum moves by s (or 2^(E-1)) against a zero
    ref0 = orc.allreduce_mean(xs0, grid, levels, bits, acc_bits, 91, 0, scale=[S])
    assert np.all(ref["sums"][planted] != ref0["sums"][planted])
    xd = [dev(x) for x in xs]
    Sd = dev(np.array([S], np.float32))
    sd = torch.empty(n, dtype=torch.int16 if acc_bits == 16 else torch.int32, device="cuda")
    g.fused_mean(xd, Sd, grid, levels, bits, 91, acc_bits, sums=sd)
    assert np.array_equal(host(sd), ref["sums"]), first_diff(host(sd), ref["sums"])
    mean = g.fused_mean(xd, Sd, grid, levels, bits, 91, acc_bits)
    assert np.array_equal(host(mean), ref["mean"]), first_diff(host(mean), ref["mean"])


@pytest.mark.parametrize("grid,world,dt", [(U, 16, "bf16"), (X, 8, "f32")])
def test_wire_quantiser_nonfinite_element(orc, grid, world, dt):
    """The wire payload's shortcut with a NaN or an infinity among small values (caller-given
    finite scale): payload bytes equal the oracle's encoding of its levels."""
    say("wire fast path non-finite", grid, world, dt)
    g = gq()
    levels = 7
    rng = np.random.default_rng(9500 + world + grid)
    n = 2 * 8192 + 333
    S = np.float32(2.1)
    inv = np.float32(np.float32(levels) / S) if grid == U else np.float32(np.float32(1.0) / S)
    bound = np.float32(1.0) if grid == U else np.float32(2.0 ** (1 - levels))
    thr = _threshold(inv, bound)
    x = (rng.standard_normal(n) * float(thr) * 0.05).astype(np.float32)
    pos = rng.choice(n, len(NONFINITE), replace=False)
    x[pos] = NONFINITE
    if dt == "bf16":
        x = _to_bf16_bits(x)
    q = orc.quantize(x, [S], grid, levels, 5, 3)
    assert np.all(np.abs(q[pos]) == levels)  # the top level (index E on the exponential grid)
    ref = orc.wire_encode(q, grid, levels, world)
    got = g.quantize_wire(dev(x), dev(np.array([S], np.float32)), grid, levels, 5, 3, world)
    assert np.array_equal(host(got), ref), first_diff(host(got), ref)


@pytest.mark.parametrize("grid,levels,bits", [(U, 7, 4), (X, 7, 4)])
@pytest.mark.parametrize("side", ["above", "below"])
def test_folded_product_at_its_scale_limit(orc, grid, levels, bits, side):
    """The 16-worker bf16 pass multiplies |x| once by the scaled inverse (inv * 2^32, or
    inv * 2^(E+31)) on the fast path, which it takes only while inv >= 2^-16, so that no
    nonzero bf16 value (the smallest is 2^-133) has a product fl(|x| * inv) that underflows to
    zero.  Scales that put inv just above that limit (fast path with subnormal products for the
    bf16 subnormals planted here) and just below it (general path) give the oracle's sums and
    means bit for bit."""
    say("folded product limit", grid, levels, side)
    g = gq()
    K = 16
    rng = np.random.default_rng(9900 + grid + (side == "below"))
    n = 2 * 8192 + 4099
    num = np.float32(levels if grid == U else 1.0)
    S = np.float32(num * np.float32(2.0 ** 16))  # inv = num / S = 2^-16 exactly
    S = np.nextafter(S, np.float32(0)) if side == "above" else np.nextafter(S, np.float32(np.inf))
    inv = np.float32(num / S)
    assert (inv >= np.float32(2.0 ** -16)) == (side == "above")
    xs = []
    for k in range(K):
        x = (rng.standard_normal(n) * float(S) * 1e-3).astype(np.float32)
        x[rng.random(n) < 0.05] = 0.0
        bits16 = (x.view(np.uint32) >> 16).astype(np.uint16)
        sub = rng.random(n) < 0.05  # bf16 subnormals of either sign, down to 2^-133
        bits16[sub] = (rng.integers(1, 0x80, sub.sum()) | (rng.integers(0, 2, sub.sum()) << 15))
        xs.append(bits16.astype(np.uint16))
    acc_bits = 16 if K * (levels if grid == U else 1 << (levels - 1)) < (1 << 15) else 32
    ref = orc.allreduce_mean(xs, grid, levels, bits, acc_bits, 123, 5, scale=[S])
    assert np.any(ref["sums"] != 0)
    xd = [dev(x) for x in xs]
    Sd = dev(np.array([S], np.float32))
    sd = torch.empty(n, dtype=torch.int16 if acc_bits == 16 else torch.int32, device="cuda")
    g.fused_mean(xd, Sd, grid, levels, bits, 123, acc_bits, index_base=5, sums=sd)
    assert np.array_equal(host(sd), ref["sums"]), first_diff(host(sd), ref["sums"])
    mean = g.fused_mean(xd, Sd, grid, levels, bits, 123, acc_bits, index_base=5)
    assert np.array_equal(host(mean), ref["mean"]), first_diff(host(mean), ref["mean"])
    # the wire payload's quantiser takes the same one-product scaling for bf16 under the same limit
    q = orc.quantize(xs[3], [S], grid, levels, 123, 3, index_base=5)
    wref = orc.wire_encode(q, grid, levels, K)
    wgot = g.quantize_wire(xd[3], Sd, grid, levels, 123, 3, K, index_base=5)
    assert np.array_equal(host(wgot), wref), first_diff(host(wgot), wref)
