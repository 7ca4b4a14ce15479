"""GPU parity of the per-worker-scale baselines (QSGD: own L2 norm; QSGDinf: own largest
magnitude; NUQSGD: exponential grid with own L2 norm) against the oracle.

Scales: the largest magnitude is exact, so bit-exact; the L2 scale sums squares in fp64 in a
different order than the oracle, so within one fp32 ulp, and bit-equal to the fp32 rounding of
the GPU's own per-worker norms from gq_global_norm.  The mean: both sides get the oracle's
scales, and since the codes are exact and the fused multiply-adds run in the same worker order,
the output is bit-exact.  Sizes span several tiles, many segments and a ragged tail; K covers
the compiled 8 and 16 and the generic loop.
"""
import numpy as np
import pytest
import torch

from allreduce_compatible_gradient_amd import workloads as W
from tests.gpu_helpers import dev, first_diff, gq, host, say

pytestmark = pytest.mark.gpu
U, X = W.UNIFORM, W.EXP


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def _np(xs):
    return [W.to_numpy(x) for x in xs]


def _check_scales(orc, g, xs_np, offsets, norm):
    xd = [dev(x) for x in xs_np]
    ref, bad = orc.worker_scales(xs_np, norm, offsets)
    got = host(g.worker_scales(xd, norm, offsets))
    assert got.shape == ref.shape
    if norm == orc.NORM_MAX:
        assert np.array_equal(got, ref), first_diff(got, ref)
    else:
        ulp = np.spacing(np.maximum(ref, np.float32(1e-38)))
        assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp), first_diff(got, ref)
        _, norms = g.global_norm(xd, offsets, norms_out=torch.empty(len(xd), ref.shape[1],
                                                                   dtype=torch.float64,
                                                                   device="cuda"))
        own = host(norms).astype(np.float32)
        own[~np.isfinite(own)] = 0.0  # a non-finite norm is stored as scale 0
        assert np.array_equal(got, own)
    return ref


def _check_mean(orc, g, xs_np, scales, grid, levels, seed, offsets=None, out_dtype=0,
                index_base=0):
    xd = [dev(x) for x in xs_np]
    ref = orc.worker_mean(xs_np, scales, grid, levels, seed, index_base, offsets, out_dtype)
    got = host(g.worker_mean(xd, dev(np.ascontiguousarray(scales, np.float32)), grid, levels,
                             seed, out_dtype, index_base, offsets))
    assert np.array_equal(got, ref), first_diff(got, ref)
    return ref


def _check_decode(orc, g, xs_np, scales, grid, levels, bits, seed, mean_ref, offsets=None,
                  out_dtype=0):
    """Receiver side: each worker's codes from gq_quantize_pack under its own scale row,
    decoded by gq_decode_workers; equal to the oracle's decode of its own codes and to the
    per-worker-scale mean."""
    n = xs_np[0].size
    off = offsets
    codes_d, codes_h = [], []
    for k, x in enumerate(xs_np):
        row = np.ascontiguousarray(scales[k], np.float32)
        cd = g.quantize_pack(dev(x), dev(row), grid, levels, bits, seed, k, 0, off)
        ch = orc.pack(orc.quantize(x, row, grid, levels, seed, k, 0, off), grid, bits)
        assert np.array_equal(host(cd), ch), first_diff(host(cd), ch)
        codes_d.append(cd)
        codes_h.append(ch)
    ref = orc.decode_workers(codes_h, n, scales, grid, levels, bits, off, out_dtype)
    got = host(g.decode_workers(codes_d, n, dev(np.ascontiguousarray(scales, np.float32)), grid,
                                levels, bits, out_dtype, off))
    assert np.array_equal(got, ref), first_diff(got, ref)
    assert np.array_equal(ref, mean_ref), first_diff(ref, mean_ref)


@pytest.mark.parametrize("name,norm,grid,levels", [
    ("flat-1.3G-f32-K8-uniform127", 0, U, 127),       # QSGD
    ("flat-1.3G-f32-K8-uniform127", 1, U, 127),       # QSGDinf
    ("resnet50-161t-f32-K8-exp7", 0, X, 7),           # NUQSGD
    ("resnet50-161t-f32-K8-exp7", 1, U, 7),
    ("gpt2s-148t-bf16-K16-uniform7", 0, U, 7),
    ("gpt2s-148t-bf16-K16-uniform7", 1, U, 7),
    ("flat-1M-f32-K4-uniform31", 0, U, 31),
])
def test_workloads(orc, name, norm, grid, levels):
    g = gq()
    w = W.reduced(name)
    say("baseline", name, norm, grid, levels)
    xs = _np(W.gradients(w, "cpu"))
    off = w.offsets if w.nseg > 1 else None
    S = _check_scales(orc, g, xs, off, norm)
    out_dtype = 1 if w.out_dtype == "bf16" else 0
    mean = _check_mean(orc, g, xs, S, grid, levels, seed=41, offsets=off, out_dtype=out_dtype)
    _check_decode(orc, g, xs, S, grid, levels, w.bits, 41, mean, off, out_dtype)


@pytest.mark.parametrize("K", [1, 3, 5, 8, 16, 17, 64])
@pytest.mark.parametrize("grid,levels", [(U, 127), (U, 3), (X, 7), (X, 12)])
def test_worker_counts_and_ragged_tail(orc, K, grid, levels):
    g = gq()
    say("baseline K", K, grid, levels)
    rng = np.random.default_rng(1000 * K + levels)
    n = 3 * 8192 + 77 if K < 64 else 8192 + 77
    xs = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-2, 1)).astype(np.float32)
          for _ in range(K)]
    S = _check_scales(orc, g, xs, None, 0)
    _check_mean(orc, g, xs, S, grid, levels, seed=7, index_base=12345)
    bits = 8 if levels > 7 else 4
    mean = _check_mean(orc, g, xs, S, grid, levels, seed=7)
    _check_decode(orc, g, xs, S, grid, levels, bits, 7, mean)


def test_bf16_inputs_and_outputs(orc):
    g = gq()
    say("baseline bf16")
    rng = np.random.default_rng(5)
    n = 2 * 8192 + 9
    xs = [((rng.standard_t(3, n) * 1e-3).astype(np.float32).view(np.uint32) >> 16)
          .astype(np.uint16) for _ in range(6)]
    S = _check_scales(orc, g, xs, None, 1)
    mean = _check_mean(orc, g, xs, S, U, 7, seed=2, out_dtype=1)
    _check_decode(orc, g, xs, S, U, 7, 4, 2, mean, out_dtype=1)
    mean = _check_mean(orc, g, xs, S, X, 7, seed=2, out_dtype=0)
    _check_decode(orc, g, xs, S, X, 7, 4, 2, mean)


def test_zero_and_unusable_workers(orc):
    """A zero worker, a worker with a non-finite element (its scale zeroed and flagged) and a
    worker whose tiny scale leaves no usable reciprocal all add nothing."""
    g = gq()
    say("baseline zero workers")
    rng = np.random.default_rng(6)
    n = 8192 + 100
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(5)]
    xs[1][:] = 0.0
    xs[2][777] = np.inf
    g.read_status()
    S = _check_scales(orc, g, xs, None, 0)
    assert g.read_status() == g.ENONFINITE
    assert S[1, 0] == 0 and S[2, 0] == 0
    S2 = S.copy()
    S2[3, 0] = np.float32(1e-45)  # s / S overflows: the worker is skipped on both sides
    _check_mean(orc, g, xs, S2, U, 31, seed=3)
    _check_mean(orc, g, xs, S2, X, 7, seed=3)


def test_nan_elements_under_a_given_scale(orc):
    """With a finite scale given by the caller a NaN element takes the top level with its sign
    bit's sign (both grids), in the baseline mean, the Global-QSGD codes and the fused pass
    alike."""
    g = gq()
    say("baseline nan")
    n = 1000
    rng = np.random.default_rng(8)
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(3)]
    xs[0][10] = np.float32(np.nan)
    xs[1][11] = np.uint32(0xFFC00000).view(np.float32)
    xs[2][12] = np.uint32(0xFF800001).view(np.float32)  # a signalling-pattern NaN, sign set
    S = np.array([[4.0], [5.0], [6.0]], np.float32)
    for grid, levels in ((U, 31), (X, 7)):
        _check_mean(orc, g, xs, S, grid, levels, seed=9)
        shared = np.array([6.0], np.float32)
        for k, x in enumerate(xs):
            ref = orc.pack(orc.quantize(x, shared, grid, levels, 9, k), grid, 8)
            got = host(g.quantize_pack(dev(x), dev(shared), grid, levels, 8, 9, k))
            assert np.array_equal(got, ref), first_diff(got, ref)
        ref = orc.allreduce_mean(xs, grid, levels, 8, 16, 9, scale=shared)
        got = host(g.fused_mean([dev(x) for x in xs], dev(shared), grid, levels, 8, 9, 16))
        assert np.array_equal(got, ref["mean"]), first_diff(got, ref["mean"])


def test_empty_and_segments(orc):
    g = gq()
    say("baseline segments")
    rng = np.random.default_rng(10)
    sizes = [0, 8, 0, 16, 8192 * 2 + 8, 0, 24, 5]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(4)]
    for norm in (0, 1):
        S = _check_scales(orc, g, xs, off, norm)
        assert np.all(S[:, [0, 2, 5]] == 0)
        mean = _check_mean(orc, g, xs, S, U, 15, seed=5, offsets=off)
        _check_decode(orc, g, xs, S, U, 15, 8, 5, mean, off)
    x0 = torch.empty(0, dtype=torch.float32, device="cuda")
    S0 = g.worker_scales([x0, x0], 0)
    assert host(S0).tolist() == [[0.0], [0.0]]
    out = g.worker_mean([x0, x0], S0, U, 7, 1)
    assert out.numel() == 0
    c0 = torch.empty(0, dtype=torch.uint8, device="cuda")
    assert g.decode_workers([c0, c0], 0, S0, U, 7, 4).numel() == 0


def test_host_checks():
    g = gq()
    say("baseline host checks")
    x = torch.zeros(16, device="cuda")
    S = torch.ones(1, 1, device="cuda")
    with pytest.raises(g.GQError) as e:
        g.worker_scales([x], norm=2)
    assert e.value.code == g.EINVAL
    with pytest.raises(g.GQError) as e:
        g.worker_mean([x], S, U, 128, 1)
    assert e.value.code == g.EINVAL
    with pytest.raises(g.GQError) as e:
        g.worker_mean([x], S, X, 31, 1)
    assert e.value.code == g.EINVAL
    with pytest.raises(g.GQError) as e:
        g.worker_mean([x] * 65, torch.ones(65, 1, device="cuda"), U, 7, 1)
    assert e.value.code == g.EINVAL
    with pytest.raises(g.GQError) as e:
        g.worker_mean([x], S, U, 7, 1, index_base=2 ** 32 - 8)
    assert e.value.code == g.EINVAL
    c = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(g.GQError) as e:
        g.decode_workers([c], 16, S, U, 8, 4)   # 8 levels do not fit 4-bit codes
    assert e.value.code == g.EINVAL
    with pytest.raises(g.GQError) as e:
        g.decode_workers([c], 16, S, U, 7, 6)
    assert e.value.code == g.EINVAL
