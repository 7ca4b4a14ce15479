"""GPU edge cases and host-side argument checks of the Global-QSGD entry points: empty and
ragged inputs, tiny segments, zero and non-finite segments, one-hot inputs at the scale, the
zero draw, the generic-K path, maximum K, and every error code the host checks return."""
import itertools

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


def _run_both(orc, xs, grid, levels, bits, acc_bits, seed=3, offsets=None, index_base=0,
              out_dtype=0):
    """Oracle path (its own scale) and GPU fused pass with the oracle's scale."""
    g = gq()
    ref = orc.allreduce_mean(xs, grid, levels, bits, acc_bits, seed, index_base, offsets,
                             out_dtype)
    xd = [dev(x) for x in xs]
    n = xs[0].size
    codes = [torch.empty(g.code_bytes(n, bits), dtype=torch.uint8, device="cuda")
             for _ in xs]
    sums = torch.empty(n, dtype=torch.int16 if acc_bits == 16 else torch.int32, device="cuda")
    S = dev(ref["scale"])
    out = g.fused_mean(xd, S, grid, levels, bits, seed, acc_bits, out_dtype, index_base,
                       offsets, codes=codes, sums=sums)
    for k in range(len(xs)):
        assert np.array_equal(host(codes[k]), ref["codes"][k]), first_diff(host(codes[k]),
                                                                          ref["codes"][k])
        q = g.quantize_pack(xd[k], S, grid, levels, bits, seed, k, index_base, offsets)
        assert np.array_equal(host(q), ref["codes"][k])
    assert np.array_equal(host(sums), ref["sums"]), first_diff(host(sums), ref["sums"])
    assert np.array_equal(host(out), ref["mean"]), first_diff(host(out), ref["mean"])
    Sg, _ = g.global_norm(xd, offsets)
    assert np.all(np.abs(host(Sg).astype(np.float64) - ref["scale"]) <= 1e-6 * ref["scale"])
    return ref


@pytest.mark.parametrize("n", [1, 7, 8, 9, 8191, 8192, 8193, 3 * 8192 + 5])
@pytest.mark.parametrize("grid,levels,bits", [(U, 7, 4), (U, 127, 8), (X, 7, 4), (X, 8, 8)])
def test_ragged_lengths(orc, n, grid, levels, bits):
    say("ragged", n, grid, levels, bits)
    rng = np.random.default_rng(n)
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(3)]
    _run_both(orc, xs, grid, levels, bits, 16)


def test_empty_buffer(orc):
    g = gq()
    say("empty")
    x = torch.empty(0, dtype=torch.float32, device="cuda")
    S, _ = g.global_norm([x, x])
    assert host(S).tolist() == [0.0]
    out = g.fused_mean([x, x], S, U, 7, 4, 1, 16)
    assert out.numel() == 0
    S2, _ = g.global_norm([x], [0, 0, 0])
    assert host(S2).tolist() == [0.0, 0.0]


def test_tiny_and_empty_segments(orc):
    say("tiny segments")
    rng = np.random.default_rng(5)
    off = [0, 8, 8, 72, 8264, 8264, 16456, 16461]
    n = off[-1]
    xs = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 1, n)).astype(np.float32)
          for _ in range(5)]
    for grid, lv, bits in ((U, 31, 8), (X, 7, 4)):
        _run_both(orc, xs, grid, lv, bits, 16, offsets=off)


def test_zero_and_nonfinite_segments(orc):
    g = gq()
    say("zero and non-finite segments")
    off = [0, 64, 128, 192]
    n = 192
    rng = np.random.default_rng(6)
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(2)]
    for x in xs:
        x[64:128] = 0.0
    xs[1][150] = np.inf
    ref = _run_both(orc, xs, U, 7, 4, 16, offsets=off)
    assert ref["scale"][1] == 0 and ref["scale"][2] == 0 and ref["nonfinite"]
    xd = [dev(x) for x in xs]
    g.read_status()
    S, _ = g.global_norm(xd, off)
    assert host(S)[2] == 0.0 and host(S)[1] == 0.0
    assert g.read_status() == g.ENONFINITE
    assert g.read_status() == g.OK
    xs[1][150] = np.nan
    _run_both(orc, xs, X, 7, 4, 16, offsets=off)
    assert g.read_status() == g.ENONFINITE


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("grid,levels,bits", [(U, 7, 4), (X, 7, 4), (U, 127, 8)])
def test_zero_and_nonfinite_segments_over_full_tiles(orc, dt, grid, levels, bits):
    """Segments whose scale is unusable (all zero; an infinite element) spanning several full
    quantisation tiles (8192 fp32 or 16384 bf16 elements): their codes are written as zero,
    also over a code buffer that held other bytes, and the segments around them stay
    bit-exact with the oracle."""
    g = gq()
    say("unusable segments over full tiles", dt, grid, levels, bits)
    tile = 8192 if dt == "f32" else 16384
    lens = [tile + 8, 3 * tile, 2 * tile + 16, tile + 5]
    off = [0] + list(np.cumsum(lens))
    n = off[-1]
    rng = np.random.default_rng(61 + grid + levels + (dt == "bf16"))
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(3)]
    for x in xs:
        x[off[1]:off[2]] = 0.0
    xs[1][off[2] + tile + 3] = np.inf
    if dt == "bf16":
        xs = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in xs]
    g.read_status()
    ref = _run_both(orc, xs, grid, levels, bits, 16, offsets=off)
    assert ref["scale"][1] == 0 and ref["scale"][2] == 0 and ref["scale"][0] > 0
    assert g.read_status() == g.ENONFINITE
    S = dev(ref["scale"])
    for k in range(len(xs)):
        codes = torch.full((g.code_bytes(n, bits),), 0xA5, dtype=torch.uint8, device="cuda")
        g.quantize_pack(dev(xs[k]), S, grid, levels, bits, 3, k, 0, off, codes=codes)
        got = host(codes)
        assert np.array_equal(got, ref["codes"][k]), first_diff(got, ref["codes"][k])
        lo, hi = off[1] * bits // 8, off[3] * bits // 8
        assert not np.any(got[lo:hi])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("base", [0, 8, 5, 4096003, "top8"])
def test_index_base_alignment(orc, dt, base):
    """The one-worker quantisers mix a part's counters once when index_base is a multiple of 8
    and element by element otherwise: codes and wire payloads equal the oracle's on both
    paths, over several full tiles and a ragged tail, on both grids."""
    g = gq()
    tile = 8192 if dt == "f32" else 16384
    n = 2 * tile + 1003
    if base == "top8":
        base = (2 ** 32 - n) // 8 * 8
    say("index base", dt, base)
    rng = np.random.default_rng(int(base) % 1000 + (dt == "bf16"))
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 0, n)).astype(np.float32)
    if dt == "bf16":
        x = (x.view(np.uint32) >> 16).astype(np.uint16)
    xd = dev(x)
    xf = x if dt == "f32" else (x.astype(np.uint32) << 16).view(np.float32)
    # the largest magnitude (levels across the range: the general path) and the L2 norm (small
    # levels: the fast path)
    scales = (np.max(np.abs(xf)), np.sqrt(np.sum(xf.astype(np.float64) ** 2)))
    for (grid, levels, bits, world), S in itertools.product(((U, 7, 4, 16), (X, 7, 4, 8),
                                                             (U, 127, 8, 8)), scales):
        Sv = np.array([S], np.float32)
        q = orc.quantize(x, Sv, grid, levels, 11, 2, index_base=base)
        codes = g.quantize_pack(xd, dev(Sv), grid, levels, bits, 11, 2, index_base=base)
        ref = orc.pack(q, grid, bits)
        assert np.array_equal(host(codes), ref), first_diff(host(codes), ref)
        pay = g.quantize_wire(xd, dev(Sv), grid, levels, 11, 2, world, index_base=base)
        ref = orc.wire_encode(q, grid, levels, world)
        assert np.array_equal(host(pay), ref), first_diff(host(pay), ref)
        assert np.any(q != 0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_store_kinds_write_the_same_bytes(orc, dt):
    """The quantisers store non-temporally when every wave store lands on whole 128-byte lines
    (line-aligned output, segments that start on lines) and through L2 otherwise.  Outputs 16
    bytes past a line and segments that start off a line take the second kind: codes and wire
    payloads equal the oracle's either way, over full tiles and ragged tails, and the bytes
    around an output are left alone."""
    g = gq()
    tile = 8192 if dt == "f32" else 16384
    n = 3 * tile + 1003
    say("store kinds", dt)
    rng = np.random.default_rng(91 + (dt == "bf16"))
    x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 0, n)).astype(np.float32)
    if dt == "bf16":
        x = (x.view(np.uint32) >> 16).astype(np.uint16)
    xd = dev(x)
    xf = x if dt == "f32" else (x.astype(np.uint32) << 16).view(np.float32)
    # one segment (on lines); segments on lines for 8-bit codes only; segments off every line
    layouts = (None, np.array([0, 2 * tile + 128, n], np.int64),
               np.array([0, 8, tile + 72, 2 * tile + 64, n], np.int64))
    for offsets, (grid, levels, bits, world) in itertools.product(
            layouts, ((U, 7, 4, 16), (X, 7, 4, 8), (U, 127, 8, 300))):
        bounds = [0, n] if offsets is None else list(offsets)
        S = np.array([np.max(np.abs(xf[b:e])) for b, e in zip(bounds[:-1], bounds[1:])],
                     np.float32)
        q = orc.quantize(x, S, grid, levels, 5, 3, offsets=offsets)
        assert np.any(q != 0)
        want = {"codes": orc.pack(q, grid, bits), "wire": orc.wire_encode(q, grid, levels, world)}
        for what, ref in want.items():
            for shift in (0, 16):
                buf = torch.full((ref.size + 256,), 0xA5, dtype=torch.uint8, device="cuda")
                base = (-buf.data_ptr()) % 128 + shift
                out = buf[base:base + ref.size]
                if what == "codes":
                    g.quantize_pack(xd, dev(S), grid, levels, bits, 5, 3, offsets=offsets,
                                    codes=out)
                else:
                    g.quantize_wire(xd, dev(S), grid, levels, 5, 3, world, offsets=offsets,
                                    payload=out)
                got = host(buf)
                assert np.array_equal(got[base:base + ref.size], ref), (
                    what, shift, first_diff(got[base:base + ref.size], ref))
                assert np.all(got[:base] == 0xA5) and np.all(got[base + ref.size:] == 0xA5)


def test_one_hot_at_scale_hits_top_level(orc):
    say("one-hot")
    n = 1000
    xs = []
    for k in range(8):
        x = np.zeros(n, np.float32)
        x[17] = (-1) ** k * 3.7
        xs.append(x)
    ref = _run_both(orc, xs, U, 127, 8, 16)
    assert ref["sums"][17] == 0  # four +127 and four -127
    xs = [np.where(np.arange(n) == 17, np.float32(2.5), np.float32(0)) for _ in range(8)]
    ref = _run_both(orc, xs, U, 127, 8, 16)
    assert ref["sums"][17] == 8 * 127


def test_zero_draw_rounds_up(orc):
    """fmix32(0) = 0: at counter == key_k the draw is exactly 0 and any p > 0 rounds up."""
    say("zero draw")
    seed = 12345
    key = orc.worker_key(seed, 0)
    n = 64
    i0 = 10
    base = (key - i0) & 0xFFFFFFFF
    if base + n > 2 ** 32:
        pytest.skip("key too close to 2^32 for this n")
    x = np.full(n, 1e-3, np.float32)
    x[0] = 1.0
    ref = _run_both(orc, [x], U, 7, 4, 16, seed=seed, index_base=base)
    assert ref["levels"][0][i0] == 1


@pytest.mark.parametrize("K", [1, 3, 5, 16, 64])
def test_worker_counts(orc, K):
    say("K", K)
    rng = np.random.default_rng(K)
    n = 20000 + K
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(K)]
    _run_both(orc, xs, U, 7, 4, 16)
    _run_both(orc, xs, X, 7, 4, 32)


def test_bf16_inputs_and_outputs(orc):
    say("bf16")
    rng = np.random.default_rng(9)
    n = 40000 + 3
    xs = [torch.from_numpy(rng.standard_t(3, n).astype(np.float32) * 1e-3).to(torch.bfloat16)
          .view(torch.int16).numpy().view(np.uint16) for _ in range(4)]
    _run_both(orc, xs, U, 7, 4, 16, out_dtype=1)
    _run_both(orc, xs, X, 7, 4, 16, out_dtype=0)


def test_denormal_and_huge_values(orc):
    say("denormal / huge")
    n = 4096
    rng = np.random.default_rng(10)
    x1 = (rng.standard_normal(n) * 1e-40).astype(np.float32)  # subnormal fp32
    x2 = (rng.standard_normal(n) * 1e30).astype(np.float32)
    for xs in ([x1, x1 * 2], [x2, x2]):
        _run_both(orc, xs, U, 31, 8, 16)
        _run_both(orc, xs, X, 7, 4, 16)


# ----------------------------------------------------------------------------- host checks
def test_argument_errors():
    g = gq()
    say("argument errors")
    x = torch.randn(64, device="cuda")
    S = torch.ones(1, device="cuda")
    codes = torch.empty(64, dtype=torch.uint8, device="cuda")

    def code_of(fn):
        with pytest.raises(g.GQError) as e:
            fn()
        return e.value.code

    assert code_of(lambda: g.quantize_pack(x, S, U, 7, 5, 1, 0)) == g.EINVAL       # bits
    assert code_of(lambda: g.quantize_pack(x, S, U, 8, 4, 1, 0)) == g.EINVAL       # s > 7
    assert code_of(lambda: g.quantize_pack(x, S, 2, 7, 4, 1, 0)) == g.EINVAL       # grid
    assert code_of(lambda: g.quantize_pack(x[1:], S, U, 7, 4, 1, 0)) == g.EALIGN   # pointer
    assert code_of(lambda: g.quantize_pack(x, S, U, 7, 4, 1, 0, offsets=[0, 4, 64])) == g.EALIGN
    assert code_of(lambda: g.quantize_pack(x, S, U, 7, 4, 1, 0, offsets=[0, 32, 60])) == g.EINVAL
    assert code_of(lambda: g.quantize_pack(x, S, U, 7, 4, 1, 0, index_base=2 ** 32 - 10)) == \
        g.EINVAL
    xs = [x] * 64
    assert code_of(lambda: g.fused_mean(xs, S, X, 10, 8, 1, 16)) == g.EOVERFLOW     # 64 * 512
    assert code_of(lambda: g.fused_mean([x] * 65, S, U, 7, 4, 1, 32)) == g.EINVAL  # K > 64
    assert code_of(lambda: g.accumulate_codes([codes] * 8, 64, U, 127, 8, 8)) == g.EINVAL
    # nothing was launched by the failed calls; a valid call still works
    out = g.fused_mean([x, x], S, U, 7, 4, 1, 16)
    assert out.shape == x.shape


@pytest.mark.parametrize("grid,levels,bits", [(U, 127, 8), (X, 7, 4)])
def test_counter_at_the_top_of_its_range(orc, grid, levels, bits):
    """index_base + n = 2^32 exactly: the last element draws counter 2^32 - 1; segments and a
    ragged end on the way, every entry point against the oracle."""
    say("counter top", grid)
    n = 3 * 8192 + 77
    base = 2 ** 32 - n
    rng = np.random.default_rng(21)
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(3)]
    off = [0, 8192, 8200, n]
    ref = _run_both(orc, xs, grid, levels, bits, 16, seed=5, offsets=off, index_base=base)
    # the fast path (no codes or sums stored) too
    g = gq()
    out = g.fused_mean([dev(x) for x in xs], dev(ref["scale"]), grid, levels, bits, 5, 16, 0,
                       base, off)
    assert np.array_equal(host(out), ref["mean"]), first_diff(host(out), ref["mean"])
