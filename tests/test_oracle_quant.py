"""Pins of the oracle's Global-QSGD path (CPU only): global norm, stochastic quantisation on
the uniform and exponential grids, packing, integer sum and decode.

Each test ties the oracle to something other than itself: closed forms, exact rational
arithmetic, a library routine, brute-force enumeration, or statistics of the definition
(unbiasedness E[Q(x)] = x from the Global-QSGD abstract's "unbiased compressor"; the QSGD
variance bound).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_layout.json")
U, X = 0, 1  # grids


def _q(orc, x, S, grid, levels, seed, worker=0, index_base=0):
    return orc.quantize(np.asarray(x, np.float32), np.asarray([S], np.float32), grid, levels,
                        seed, worker, index_base)


# ----------------------------------------------------------------------------- zero
def test_zero_vector_maps_to_zero(orc):
    xs = [np.zeros(100, np.float32) for _ in range(3)]
    res = orc.allreduce_mean(xs, U, 7, 4, 16, seed=1)
    assert res["scale"][0] == 0.0
    assert not res["nonfinite"]
    for q in res["levels"]:
        assert not q.any()
    assert not res["sums"].any()
    assert not res["mean"].any()
    res = orc.allreduce_mean(xs, X, 7, 4, 16, seed=1)
    assert not res["mean"].any()


def test_zero_segment_among_nonzero(orc):
    rng = np.random.default_rng(0)
    off = [0, 16, 48, 64]
    xs = [rng.standard_normal(64).astype(np.float32) for _ in range(2)]
    for x in xs:
        x[16:48] = 0.0
    res = orc.allreduce_mean(xs, U, 31, 8, 32, seed=3, offsets=off)
    assert res["scale"][1] == 0.0 and res["scale"][0] > 0 and res["scale"][2] > 0
    assert not res["sums"][16:48].any()
    assert res["sums"][:16].any()


def test_negative_zero_and_sign_of_zero_level(orc):
    S = np.float32(1.0)
    assert orc.quant_one(U, 7, -0.0, S, 123, 5) == 0
    # tiny negative value on the exponential grid that rounds down: code is 0, not "-0"
    key = orc.worker_key(1, 0)
    for c in range(200):
        q = orc.quant_one(X, 7, -1e-30, S, key, c)
        assert q in (0, -1)
    assert orc.pack([0], X, 4)[0] == 0


# ----------------------------------------------------------------------------- range
@pytest.mark.parametrize("s", [1, 7, 31, 127])
def test_code_range_one_hot_at_scale(orc, s):
    rng = np.random.default_rng(s)
    hit_above = False
    for t in range(400):
        a = np.float32(rng.uniform(1e-3, 1e3) * (1 if t % 2 else -1))
        x = np.zeros(8, np.float32)
        x[t % 8] = a
        S, _, _ = orc.global_norm([x])
        assert S[0] == abs(a)
        u = np.float32(abs(a)) * (np.float32(s) / S[0])
        hit_above |= bool(u > s)
        q = _q(orc, x, S[0], U, s, seed=t)
        assert np.abs(q).max() <= s
        assert q[t % 8] == (s if a > 0 else -s)
    if s > 1:  # a * fl(1/a) never exceeds 1 in fp32, so s = 1 cannot reach the clamp
        assert hit_above, "no case exercised the clamp above the top level"


def test_code_never_exceeds_s_when_u_rounds_above(orc):
    """|x| = S can give u = fl(|x| * fl(s/S)) one ulp above s; the top level must still be s.
    2^21 elements at such a scale make an unclamped round-up (probability u - s per element,
    about 2^-17) all but certain to show."""
    s = 127
    rng = np.random.default_rng(5)
    S = rng.uniform(1.0, 2.0, 400000).astype(np.float32)
    u = (S * (np.float32(s) / S)).astype(np.float32)
    S = S[np.argmax(u)]
    assert u.max() > s
    x = np.full(1 << 21, S, np.float32)
    x[1::2] = -S
    q = orc.quantize(x, [S], U, s, seed=3, worker=0)
    assert q.max() == s and q.min() == -s


def test_exp_code_range(orc):
    rng = np.random.default_rng(1)
    for E in (1, 3, 7):
        x = rng.standard_normal(200).astype(np.float32) * np.float32(10) ** rng.uniform(
            -8, 2, 200).astype(np.float32)
        S, _, _ = orc.global_norm([x])
        for seed in range(5):
            q = _q(orc, x, S[0], X, E, seed)
            assert np.abs(q).max() <= E


# ----------------------------------------------------------------------------- overflow
def test_worst_case_sums_are_exact(orc):
    K, s, n = 8, 127, 32
    for sign in (1, -1):
        xs = []
        for k in range(K):
            x = np.zeros(n, np.float32)
            x[5] = sign * 3.0
            xs.append(x)
        res = orc.allreduce_mean(xs, U, s, 8, 16, seed=9)
        assert res["sums"][5] == sign * K * s
        assert res["overflow"] == 0
        assert res["mean"][5] == np.float32(sign * 3.0)


def test_accumulator_overflow_is_reported(orc):
    # 259 workers at level 127 exceed int16 (259 * 127 = 32893 > 32767)
    codes = [orc.pack(np.full(4, 127, np.int32), U, 8)] * 259
    _, over = orc.accumulate(codes, 4, U, 8, 16)
    assert over == 4
    _, over = orc.accumulate(codes[:258], 4, U, 8, 16)
    assert over == 0
    # and below: 259 workers at level -127 give -32893 < -32768
    neg = [orc.pack(np.full(4, -127, np.int32), U, 8)] * 259
    _, over = orc.accumulate(neg, 4, U, 8, 16)
    assert over == 4
    sums, over = orc.accumulate(neg[:258], 4, U, 8, 16)
    assert over == 0 and sums[0] == -258 * 127


# ----------------------------------------------------------------------------- exact levels
@pytest.mark.parametrize("s", [7, 31, 127])
@pytest.mark.parametrize("k", [-3, 0, 5])
def test_exact_uniform_levels_round_trip(orc, s, k):
    j = np.arange(-s, s + 1, dtype=np.int32)
    x = (j * 2.0 ** k).astype(np.float32)
    S = np.float32(s * 2.0 ** k)
    for seed in range(8):
        q = _q(orc, x, S, U, s, seed)
        assert np.array_equal(q, j)
        sums = q.astype(np.int32)
        mean = orc.dequantize(sums, [S], U, s, 1)
        assert np.array_equal(mean, x)


@pytest.mark.parametrize("E", [1, 3, 7])
def test_exact_exponential_levels_round_trip(orc, E):
    S = np.float32(2.0 ** 5)
    j = np.arange(-E, E + 1, dtype=np.int32)
    mag = np.where(j == 0, 0.0, 2.0 ** (np.abs(j) - E))
    x = (np.sign(j) * mag * S).astype(np.float32)
    for seed in range(8):
        q = _q(orc, x, S, X, E, seed)
        assert np.array_equal(q, j)
        sums = np.array([orc.lin(X, int(v)) for v in q], np.int32)
        mean = orc.dequantize(sums, [S], X, E, 1)
        assert np.array_equal(mean, x)


# ----------------------------------------------------------------------------- identity
def test_allreduce_compatibility_identity(orc):
    """Summing the codes and decoding once equals the mean of the per-worker decodes."""
    rng = np.random.default_rng(5)
    K, n = 4, 512
    xs = [(rng.standard_normal(n) * (k + 1)).astype(np.float32) for k in range(K)]
    for grid, lv, bits in ((U, 31, 8), (U, 7, 4), (X, 7, 4)):
        res = orc.allreduce_mean(xs, grid, lv, bits, 32, seed=11)
        S = float(res["scale"][0])
        unit = 1.0 / lv if grid == U else 2.0 ** (1 - lv)
        per = [np.array([orc.lin(grid, int(v)) for v in q], np.float64) * unit * S
               for q in res["levels"]]
        ref = np.mean(per, axis=0)
        err = np.abs(res["mean"].astype(np.float64) - ref)
        assert err.max() <= 2 * np.finfo(np.float32).eps * max(np.abs(ref).max(), S / K)


def test_per_worker_scales_break_summability(orc):
    """Negative control: QSGD with each worker's own norm is not allreduce-compatible."""
    rng = np.random.default_rng(6)
    K, n, s = 4, 256, 31
    xs = [(rng.standard_normal(n) * 4.0 ** k).astype(np.float32) for k in range(K)]
    norms = [np.float32(np.linalg.norm(x.astype(np.float64))) for x in xs]
    q = [_q(orc, x, norms[k], U, s, seed=2, worker=k) for k, x in enumerate(xs)]
    true = np.mean([q[k] * float(norms[k]) / s for k in range(K)], axis=0)
    # summing codes then decoding with any one shared scale is far off
    summed = np.sum(q, axis=0)
    best = min(np.abs(summed * float(S) / (s * K) - true).max() for S in norms)
    assert best > 100 * np.finfo(np.float32).eps * np.abs(true).max()


# ----------------------------------------------------------------------------- statistics
def _exact_moments_uniform(x, S, s):
    u = np.minimum(np.abs(x.astype(np.float32)) * np.float32(np.float32(s) / np.float32(S)),
                   np.float32(s)).astype(np.float64)
    p = u - np.floor(u)
    step = float(S) / s
    return p, step * step * p * (1 - p)


def test_unbiasedness_uniform_monte_carlo(orc):
    rng = np.random.default_rng(7)
    d, s, N = 16, 7, 20000
    x = rng.standard_normal(d).astype(np.float32)
    S = np.float32(np.linalg.norm(x.astype(np.float64)))
    acc = np.zeros(d)
    sq = np.zeros(d)
    for seed in range(N):
        v = _q(orc, x, S, U, s, seed).astype(np.float64) * float(S) / s
        acc += v
        sq += (v - x.astype(np.float64)) ** 2
    mean = acc / N
    p, var = _exact_moments_uniform(x, S, s)
    z = (mean - x.astype(np.float64)) / np.sqrt(np.maximum(var, 1e-300) / N)
    assert np.all(np.abs(z[var > 0]) < 5)
    assert np.all(mean[var == 0] == x[var == 0])
    # the Monte Carlo squared error matches the exact two-point variance; the squared error
    # of one draw has variance step^4 p (1-p) (1-2p)^2
    step = float(S) / s
    sd = np.sqrt((step ** 4 * p * (1 - p) * (1 - 2 * p) ** 2).sum() / N)
    assert abs(sq.sum() / N - var.sum()) < 5 * sd


def test_unbiasedness_exponential_monte_carlo(orc):
    rng = np.random.default_rng(8)
    d, E, N = 16, 7, 20000
    x = (rng.laplace(size=d) * 10.0 ** rng.uniform(-2, 0, d)).astype(np.float32)
    S = np.float32(np.linalg.norm(x.astype(np.float64)))
    acc = np.zeros(d)
    for seed in range(N):
        q = _q(orc, x, S, X, E, seed)
        acc += np.array([orc.lin(X, int(v)) for v in q], np.float64)
    mean = acc / N * 2.0 ** (1 - E) * float(S)
    # exact variance of the two-point law between neighbouring levels
    u = np.minimum(np.abs(x) * np.float32(np.float32(1) / S), np.float32(1)).astype(np.float64)
    lv = np.concatenate([[0.0], 2.0 ** (np.arange(1, E + 1) - E)])
    j = np.searchsorted(lv, u, side="right") - 1
    lo = lv[j]
    hi = lv[np.minimum(j + 1, E)]
    gap = np.where(j == E, 0.0, hi - lo)
    p = np.where(gap > 0, (u - lo) / np.where(gap > 0, gap, 1), 0.0)
    var = (gap * float(S)) ** 2 * p * (1 - p)
    z = (mean - x.astype(np.float64)) / np.sqrt(np.maximum(var, 1e-300) / N)
    assert np.all(np.abs(z[var > 0]) < 5)


def test_qsgd_variance_bound(orc):
    """Exact variance sum (S/s)^2 p(1-p) is within min(d/s^2, sqrt(d)/s * |x|/S) S^2, which at
    S = |x| is QSGD's min(d/s^2, sqrt(d)/s) |x|^2."""
    rng = np.random.default_rng(9)
    for t in range(300):
        d = int(rng.integers(1, 64))
        s = int(rng.choice([1, 3, 7, 31, 127]))
        x = (rng.standard_normal(d) * 10.0 ** rng.uniform(-3, 3, d)).astype(np.float32)
        nrm = np.float32(np.linalg.norm(x.astype(np.float64)))
        S = nrm * np.float32(1 + rng.uniform(0, 3) * (t % 2))  # half at S = |x|, half above
        _, var = _exact_moments_uniform(x, S, s)
        total = var.sum()
        bound = min(d / s ** 2, math.sqrt(d) / s * float(nrm) / float(S)) * float(S) ** 2
        assert total <= bound * (1 + 1e-6)
        if S == nrm:
            assert total <= min(d / s ** 2, math.sqrt(d) / s) * float(nrm) ** 2 * (1 + 1e-6)


def test_brute_force_joint_distribution(orc):
    """d = 4: all 2^4 round-up patterns against their product-Bernoulli probabilities."""
    from scipy import stats
    x = np.array([0.3, -1.7, 2.25, -0.05], np.float32)
    S, s, N = np.float32(4.0), 2, 100000
    u = np.abs(x) * np.float32(np.float32(s) / S)
    lo = np.floor(u).astype(np.int64)
    p = (u - lo).astype(np.float64)
    counts = {}
    for seed in range(N):
        q = np.abs(_q(orc, x, S, U, s, seed)) - lo
        assert set(q.tolist()) <= {0, 1}
        key = tuple(q.tolist())
        counts[key] = counts.get(key, 0) + 1
    obs, exp = [], []
    for pat in itertools.product((0, 1), repeat=4):
        pr = np.prod([p[i] if b else 1 - p[i] for i, b in enumerate(pat)])
        obs.append(counts.get(pat, 0))
        exp.append(pr * N)
    obs, exp = np.array(obs), np.array(exp)
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert stats.chi2.sf(chi2, 15) > 1e-4


def test_round_up_when_draw_is_zero(orc):
    # fmix32(0) = 0: the counter equal to the key draws r = 0 < p for any p > 0
    key = orc.worker_key(4, 2)
    assert orc.quant_one(U, 7, 1e-30, 1.0, key, key) == 1
    assert orc.quant_one(X, 7, 1e-30, 1.0, key, key) == 1
    assert orc.quant_one(U, 7, 0.0, 1.0, key, key) == 0


# ----------------------------------------------------------------------------- global norm
def test_global_norm_closed_forms(orc):
    d = 4 ** 6
    for c in (0.5, -3.0, 2.0 ** -20):
        S, norms, _ = orc.global_norm([np.full(d, c, np.float32)])
        assert norms[0, 0] == abs(c) * 2 ** 6
    x = np.zeros(1000, np.float32)
    x[123] = -7.25
    S, norms, _ = orc.global_norm([x])
    assert S[0] == np.float32(7.25)


def test_global_norm_against_exact_sum(orc):
    rng = np.random.default_rng(10)
    off = [0, 1000, 1001, 5000, 12000]
    xs = [(rng.standard_normal(12000) * 10.0 ** rng.uniform(-3, 3, 12000)).astype(np.float32)
          for _ in range(3)]
    S, norms, bad = orc.global_norm(xs, off)
    assert not bad
    for g in range(4):
        ref = [math.sqrt(math.fsum(float(v) ** 2 for v in x[off[g]:off[g + 1]])) for x in xs]
        for k in range(3):
            assert abs(norms[k, g] - ref[k]) <= 1e-12 * ref[k]
        assert S[g] == np.float32(max(ref))


def test_global_norm_bf16(orc):
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal(4096).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    S, norms, _ = orc.global_norm([bits])
    ref = math.sqrt(math.fsum(float(v) ** 2 for v in x.float().numpy()))
    assert abs(norms[0, 0] - ref) <= 1e-12 * ref


def test_global_norm_nonfinite_zeroes_segment(orc):
    x = np.ones(64, np.float32)
    y = np.ones(64, np.float32)
    y[40] = np.inf
    S, _, bad = orc.global_norm([x, y], [0, 32, 64])
    assert bad
    assert S[0] == np.float32(math.sqrt(32)) and S[1] == 0.0
    y[40] = np.nan
    S, _, bad = orc.global_norm([x, y], [0, 32, 64])
    assert bad and S[1] == 0.0


def test_streamed_global_norm_equals_whole(orc):
    """Sums of squares chained chunk by chunk and finished by norm_finish give global_norm's
    result bit for bit (the full-size GPU parity streams 41.6 GB this way), and the finish
    against exact sums stays within the same 1e-12 as the whole-buffer form."""
    rng = np.random.default_rng(13)
    off = [0, 5000, 5000, 70001, 100003]
    xs = [(rng.standard_normal(100003) * 10.0 ** rng.uniform(-3, 3, 100003)).astype(np.float32)
          for _ in range(3)]
    S, norms, bad = orc.global_norm(xs, off)
    ss = np.zeros((3, 4))
    for k, x in enumerate(xs):
        for g in range(4):
            acc = 0.0
            for c in range(off[g], off[g + 1], 777):
                acc = orc.sumsq(x[c:min(c + 777, off[g + 1])], acc)
            ss[k, g] = acc
    S2, norms2, bad2 = orc.norm_finish(ss)
    assert np.array_equal(S, S2) and np.array_equal(norms, norms2) and bad == bad2 == False
    for g in (0, 2, 3):
        ref = max(math.sqrt(math.fsum(float(v) ** 2 for v in x[off[g]:off[g + 1]])) for x in xs)
        assert S2[g] == np.float32(ref)
    assert S2[1] == 0.0
    ss[1, 2] = np.inf
    S3, _, bad3 = orc.norm_finish(ss)
    assert bad3 and S3[2] == 0.0 and S3[0] == S[0]


# ----------------------------------------------------------------------------- decode
def test_decode_factor_exact_rational(orc):
    rng = np.random.default_rng(12)
    for _ in range(2000):
        S = np.float32(10.0 ** rng.uniform(-30, 30))
        K = int(rng.integers(1, 65))
        grid = int(rng.integers(0, 2))
        lv = int(rng.integers(1, 128)) if grid == U else int(rng.integers(1, 8))
        D = lv * K if grid == U else K * 2 ** (lv - 1)
        want = np.float32(float(Fraction(float(S)) / D))
        assert orc.decode_factor(grid, lv, K, S) == want
    assert orc.decode_factor(U, 7, 2, 0.0) == 0.0
    assert orc.decode_factor(U, 7, 2, float("inf")) == 0.0


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(13)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    # ties, just-below/above ties, near-overflow and subnormals
    extra = []
    for hi in (0x3F80, 0x3F81, 0x7F7F, 0x0001, 0x8001, 0xC2AB):
        for lo in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF):
            extra.append((hi << 16) | lo)
    bits = np.concatenate([bits, np.array(extra, np.uint32)])
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(v) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------------------- codes
def test_pack_layout_golden(orc):
    for case in json.load(open(GOLDEN))["cases"]:
        grid = U if case["grid"] == "uniform" else X
        got = orc.pack(np.array(case["levels"], np.int32), grid, case["bits"])
        assert got.tolist() == case["bytes"], case
        back = orc.unpack(got, len(case["levels"]), grid, case["bits"])
        assert back.tolist() == case["levels"]


def test_exponential_linear_values(orc):
    assert orc.lin(X, 0) == 0
    for j in range(1, 8):
        assert orc.lin(X, j) == 2 ** (j - 1)
        assert orc.lin(X, -j) == -(2 ** (j - 1))
    for q in range(-127, 128):
        assert orc.lin(U, q) == q


def test_counter_offset_chunking_is_consistent(orc):
    rng = np.random.default_rng(14)
    x = rng.standard_normal(1000).astype(np.float32)
    S = np.float32(np.linalg.norm(x))
    whole = _q(orc, x, S, U, 31, seed=5, worker=3)
    part = _q(orc, x[600:], S, U, 31, seed=5, worker=3, index_base=600)
    assert np.array_equal(whole[600:], part)


def test_quantize_list_matches_buffer_form(orc):
    rng = np.random.default_rng(15)
    x = rng.standard_normal(300).astype(np.float32)
    S = np.float32(np.linalg.norm(x))
    whole = _q(orc, x, S, X, 7, seed=8, worker=2, index_base=17)
    idx = rng.choice(300, 50, replace=False)
    got = orc.quantize_list(x[idx], np.full(50, S), idx + 17, X, 7, orc.worker_key(8, 2))
    assert np.array_equal(got, whole[idx])


def test_mean_is_unbiased_end_to_end(orc):
    rng = np.random.default_rng(16)
    K, d, N = 3, 8, 4000
    xs = [rng.standard_normal(d).astype(np.float32) for _ in range(K)]
    true = np.mean([x.astype(np.float64) for x in xs], axis=0)
    acc = np.zeros(d)
    for seed in range(N):
        acc += orc.allreduce_mean(xs, U, 3, 4, 16, seed)["mean"]
    S = max(np.linalg.norm(x.astype(np.float64)) for x in xs)
    sd = S / 3 / 2 / math.sqrt(K) / math.sqrt(N)  # each worker's rounding sd <= step/2
    assert np.all(np.abs(acc / N - true) < 5 * sd)


def test_nan_goes_to_the_top_level(orc):
    """Under a caller-given finite scale a NaN element is clamped to the top level with the
    sign its sign bit gives it, on both grids (the pages say nothing of NaN: a reading; the
    sign bit is IEEE 754's sign of every value, NaN included)."""
    pos = np.float32(np.nan)
    neg = np.uint32(0xFFC00000).view(np.float32)
    x = np.array([pos, neg, 1.0, -1.0], np.float32)
    for seed in range(5):
        q = _q(orc, x, 4.0, U, 31, seed)
        assert q[0] == 31 and q[1] == -31
        q = _q(orc, x, 4.0, X, 7, seed)
        assert q[0] == 7 and q[1] == -7
