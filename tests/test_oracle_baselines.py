"""Pins of the oracle's per-worker-scale baselines (CPU only): QSGD (each worker's own L2 norm),
QSGDinf (read as each worker's own largest magnitude) and NUQSGD (exponential grid, own L2
norm), whose codes are not summable, so the receiver decodes every worker with that worker's
scale.  The NUQSGD abstract names QSGD and QSGDinf as the baselines of the family.

Each test ties the oracle to something other than itself: numpy's norm and maximum, exact
rational arithmetic where the decode factors are powers of two, exact level values,
unbiasedness over seeds, and QSGD's variance bound for the mean of independent workers.
"""
from fractions import Fraction

import numpy as np
import pytest

U, X = 0, 1  # grids


def _segments(rng, n, nseg):
    cuts = np.sort(rng.choice(np.arange(1, n), nseg - 1, replace=False))
    return np.concatenate([[0], cuts, [n]]).astype(np.int64)


# ----------------------------------------------------------------------------- scales
@pytest.mark.parametrize("bf16", [False, True])
def test_l2_scales_against_numpy(orc, bf16):
    rng = np.random.default_rng(21)
    K, n = 3, 5000
    off = _segments(rng, n, 7)
    xs = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 2, n)).astype(np.float32)
          for _ in range(K)]
    if bf16:
        xs = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in xs]
    S, bad = orc.worker_scales(xs, orc.NORM_L2, off)
    assert not bad and S.shape == (K, 7)
    for k, x in enumerate(xs):
        v = (x.astype(np.uint32) << 16).view(np.float32) if bf16 else x
        for g in range(7):
            ref = np.linalg.norm(v[off[g]:off[g + 1]].astype(np.float64))
            # fp64 sums in different orders agree far below fp32's resolution
            assert abs(float(S[k, g]) - ref) <= 0.51 * np.spacing(np.float32(ref)), (k, g)


@pytest.mark.parametrize("bf16", [False, True])
def test_max_scales_are_numpy_maximum(orc, bf16):
    rng = np.random.default_rng(22)
    K, n = 4, 3001
    off = _segments(rng, n, 5)
    xs = [(rng.laplace(size=n) * 10.0 ** rng.uniform(-4, 1, n)).astype(np.float32)
          for _ in range(K)]
    if bf16:
        xs = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in xs]
    S, bad = orc.worker_scales(xs, orc.NORM_MAX, off)
    assert not bad
    for k, x in enumerate(xs):
        v = (x.astype(np.uint32) << 16).view(np.float32) if bf16 else x
        for g in range(5):
            assert S[k, g] == np.abs(v[off[g]:off[g + 1]]).max(), (k, g)


@pytest.mark.parametrize("norm", [0, 1])
@pytest.mark.parametrize("bad_value", [np.nan, np.inf, -np.inf])
def test_nonfinite_scale_is_zeroed_and_reported(orc, norm, bad_value):
    rng = np.random.default_rng(23)
    off = np.array([0, 40, 100], np.int64)
    xs = [rng.standard_normal(100).astype(np.float32) for _ in range(3)]
    clean, bad = orc.worker_scales(xs, norm, off)
    assert not bad and np.all(clean > 0)
    xs[1][57] = bad_value
    S, bad = orc.worker_scales(xs, norm, off)
    assert bad
    assert S[1, 1] == 0.0
    mask = np.ones_like(S, bool)
    mask[1, 1] = False
    assert np.array_equal(S[mask], clean[mask])


def test_l2_overflow_to_infinity_is_reported(orc):
    x = np.full(8, 3e38, np.float32)  # finite elements, norm above the fp32 range
    S, bad = orc.worker_scales([x], orc.NORM_L2)
    assert bad and S[0, 0] == 0.0
    S, bad = orc.worker_scales([x], orc.NORM_MAX)
    assert not bad and S[0, 0] == np.float32(3e38)


def test_zero_worker_has_zero_scale(orc):
    xs = [np.ones(10, np.float32), np.zeros(10, np.float32)]
    for norm in (0, 1):
        S, bad = orc.worker_scales(xs, norm)
        assert not bad and S[1, 0] == 0.0 and S[0, 0] > 0


# ----------------------------------------------------------------------------- mean
def _exact_mean_pow2(orc, xs, scales, grid, levels, seed, off):
    """Exact rational mean when every decode factor is a power of two: the levels come from
    orc.quantize (pinned on its own), each decoded with its own worker's factor."""
    K = len(xs)
    n = xs[0].size
    out = [Fraction(0)] * n
    for k, x in enumerate(xs):
        q = orc.quantize(x, scales[k], grid, levels, seed, k, 0, off)
        for g in range(off.size - 1):
            S = Fraction(float(scales[k, g]))
            D = levels * K if grid == U else K * 2 ** (levels - 1)
            f = S / D
            for i in range(off[g], off[g + 1]):
                out[i] += orc.lin(grid, int(q[i])) * f
    return out


@pytest.mark.parametrize("grid,levels", [(U, 7), (U, 127), (X, 7)])
def test_power_of_two_factors_give_the_exact_mean(orc, grid, levels):
    """S_{k,g} = D * 2^e_{k,g} makes every product and partial sum exact in fp32, so the mean
    must be the exact rational one; distinct exponents per worker catch a scale taken from
    the wrong worker or segment."""
    rng = np.random.default_rng(24)
    K, n = 5, 600
    off = _segments(rng, n, 4)
    D = levels * K if grid == U else K * 2 ** (levels - 1)
    e = rng.integers(-14, -6, size=(K, 4))
    scales = (D * np.exp2(e.astype(np.float64))).astype(np.float32)
    xs = []
    for k in range(K):
        x = np.empty(n, np.float32)
        for g in range(4):
            seg = slice(off[g], off[g + 1])
            x[seg] = rng.uniform(-1, 1, off[g + 1] - off[g]) * float(scales[k, g])
        xs.append(x)
    got = orc.worker_mean(xs, scales, grid, levels, seed=31, offsets=off)
    exact = _exact_mean_pow2(orc, xs, scales, grid, levels, 31, off)
    assert all(Fraction(float(got[i])) == exact[i] for i in range(n))


def test_one_worker_equals_the_global_path(orc):
    """K = 1: the worker's own scale is the global one, and fma(l, f, 0) = fp32(l * f)."""
    rng = np.random.default_rng(25)
    off = _segments(rng, 4000, 6)
    for grid, levels, bits in ((U, 31, 8), (U, 7, 4), (X, 7, 4)):
        x = (rng.standard_normal(4000) * 3).astype(np.float32)
        S, _ = orc.worker_scales([x], orc.NORM_L2, off)
        ref = orc.allreduce_mean([x], grid, levels, bits, 32, 9, 0, off, scale=S[0])
        got = orc.worker_mean([x], S, grid, levels, 9, offsets=off)
        assert np.array_equal(got, ref["mean"])


def test_zero_and_invalid_workers_contribute_nothing(orc):
    """A worker whose scale is 0 (zero data, or a zeroed non-finite norm) adds 0; with
    power-of-two factors the others' sum is exact, over K (the zero worker still counts)."""
    rng = np.random.default_rng(26)
    K, n, s = 3, 200, 15
    off = np.array([0, n], np.int64)
    scales = np.array([[s * K * 2.0 ** -8], [0.0], [s * K * 2.0 ** -5]], np.float32)
    xs = [rng.uniform(-1, 1, n).astype(np.float32) * float(scales[k, 0]) for k in range(K)]
    xs[1] = rng.standard_normal(n).astype(np.float32)  # ignored: its scale is 0
    got = orc.worker_mean(xs, scales, U, s, seed=4, offsets=off)
    exact = _exact_mean_pow2(orc, [xs[0], np.zeros(n, np.float32), xs[2]], scales, U, s, 4, off)
    assert all(Fraction(float(got[i])) == exact[i] for i in range(n))


@pytest.mark.parametrize("grid,levels", [(U, 5), (X, 6)])
def test_exact_levels_are_deterministic(orc, grid, levels):
    """Values on a worker's own grid are reproduced whatever the seed."""
    rng = np.random.default_rng(27)
    K, n = 3, 64
    scales = np.array([[2.0], [0.75], [5.0]], np.float32)
    xs = []
    for k in range(K):
        if grid == U:
            lv = rng.integers(-levels, levels + 1, n)
            xs.append((lv * (float(scales[k, 0]) / levels)).astype(np.float32))
        else:
            j = rng.integers(0, levels + 1, n)
            sign = rng.choice([-1.0, 1.0], n)
            xs.append((sign * np.where(j == 0, 0.0, 2.0 ** (j - levels)) *
                       float(scales[k, 0])).astype(np.float32))
    # the grid values above are exact in fp32 when S/levels is; check and then compare seeds
    outs = [orc.worker_mean(xs, scales, grid, levels, seed) for seed in (1, 2, 3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    true = np.mean(np.stack(xs).astype(np.float64), axis=0)
    assert np.allclose(outs[0], true, rtol=1e-6, atol=1e-7)


def test_max_scale_puts_a_power_of_two_peak_on_the_top_level(orc):
    """QSGDinf: the element of largest magnitude, when it is a power of two, lands exactly on
    level +-s (u = s with no rounding)."""
    rng = np.random.default_rng(28)
    s = 127
    for t in range(20):
        x = rng.uniform(-0.49, 0.49, 100).astype(np.float32) * np.float32(2.0 ** (t - 10))
        i = int(rng.integers(0, 100))
        x[i] = np.float32((-1) ** t * 2.0 ** (t - 10))
        S, _ = orc.worker_scales([x], orc.NORM_MAX)
        assert S[0, 0] == abs(x[i])
        q = orc.quantize(x, S[0], U, s, seed=t, worker=0)
        assert q[i] == (-1) ** t * s
        assert np.all(np.abs(q) <= s)


# ----------------------------------------------------------------------------- statistics
def test_mean_is_unbiased_over_seeds(orc):
    rng = np.random.default_rng(29)
    K, d, s, N = 4, 12, 3, 6000
    xs = [(rng.standard_normal(d) * 2.0 ** k).astype(np.float32) for k in range(K)]
    for norm in (orc.NORM_L2, orc.NORM_MAX):
        S, _ = orc.worker_scales(xs, norm)
        acc = np.zeros(d)
        for seed in range(N):
            acc += orc.worker_mean(xs, S, U, s, seed).astype(np.float64)
        mean = acc / N
        # exact variance of the mean: sum over workers of (S_k/(sK))^2 p(1-p)
        var = np.zeros(d)
        for k, x in enumerate(xs):
            u = np.minimum(np.abs(x) * np.float32(np.float32(s) / S[k, 0]),
                           np.float32(s)).astype(np.float64)
            p = u - np.floor(u)
            var += (float(S[k, 0]) / (s * K)) ** 2 * p * (1 - p)
        true = np.mean(np.stack(xs).astype(np.float64), axis=0)
        z = (mean - true) / np.sqrt(np.maximum(var, 1e-300) / N)
        assert np.all(np.abs(z[var > 0]) < 5), norm


def test_qsgd_variance_bound_for_the_mean(orc):
    """With each worker at its own L2 norm, E|mean - true|^2 is at most
    sum_k min(d/s^2, sqrt(d)/s) |x_k|^2 / K^2 (QSGD's bound for independent workers);
    the Monte Carlo estimate stays under it."""
    rng = np.random.default_rng(30)
    K, d, s, N = 3, 20, 2, 3000
    xs = [(rng.standard_normal(d) * 10.0 ** rng.uniform(-1, 1, d)).astype(np.float32)
          for _ in range(K)]
    S, _ = orc.worker_scales(xs, orc.NORM_L2)
    true = np.mean(np.stack(xs).astype(np.float64), axis=0)
    err = 0.0
    for seed in range(N):
        err += ((orc.worker_mean(xs, S, U, s, seed).astype(np.float64) - true) ** 2).sum()
    err /= N
    bound = sum(min(d / s ** 2, np.sqrt(d) / s) * float(np.linalg.norm(x.astype(np.float64))) ** 2
                for x in xs) / K ** 2
    assert err <= bound


def test_bf16_output_is_the_rounded_fp32_mean(orc):
    rng = np.random.default_rng(31)
    xs = [rng.standard_normal(300).astype(np.float32) for _ in range(4)]
    S, _ = orc.worker_scales(xs, orc.NORM_L2)
    f = orc.worker_mean(xs, S, U, 7, 3)
    b = orc.worker_mean(xs, S, U, 7, 3, out_dtype=orc.BF16)
    import torch
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


# ----------------------------------------------------------------------------- receiver
@pytest.mark.parametrize("grid,levels,bits", [(U, 7, 4), (U, 127, 8), (X, 7, 4), (X, 8, 8)])
def test_decoding_codes_gives_the_exact_mean(orc, grid, levels, bits):
    """The receiver's decode of packed codes with power-of-two factors is the exact rational
    mean of the levels; distinct exponents per worker and segment catch a wrong factor."""
    rng = np.random.default_rng(32)
    K, n = 4, 301
    off = _segments(rng, n, 3)
    D = levels * K if grid == U else K * 2 ** (levels - 1)
    e = rng.integers(-12, -4, size=(K, 3))
    scales = (D * np.exp2(e.astype(np.float64))).astype(np.float32)
    xs = [np.empty(n, np.float32) for _ in range(K)]
    for k in range(K):
        for g in range(3):
            seg = slice(off[g], off[g + 1])
            xs[k][seg] = rng.uniform(-1, 1, off[g + 1] - off[g]) * float(scales[k, g])
    codes = [orc.pack(orc.quantize(x, scales[k], grid, levels, 17, k, 0, off), grid, bits)
             for k, x in enumerate(xs)]
    got = orc.decode_workers(codes, n, scales, grid, levels, bits, off)
    exact = _exact_mean_pow2(orc, xs, scales, grid, levels, 17, off)
    assert all(Fraction(float(got[i])) == exact[i] for i in range(n))


def test_codes_of_an_unusable_scale_add_nothing(orc):
    """A worker whose scale is 0 has decode factor 0: even nonzero codes add nothing."""
    n, s = 64, 7
    codes = [orc.pack(np.full(n, 3, np.int32), U, 8), orc.pack(np.full(n, -5, np.int32), U, 8)]
    scales = np.array([[2.0 * s * 2], [0.0]], np.float32)  # factor of worker 0: 2^1
    got = orc.decode_workers(codes, n, scales, U, s, 8)
    assert np.all(got == 6.0)
