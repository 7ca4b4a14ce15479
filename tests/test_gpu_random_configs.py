"""Seeded random configurations through every Global-QSGD and baseline entry point, each
compared with the oracle: lengths (ragged, tile-crossing), segment layouts (empty and tiny
segments), worker counts (compiled and generic paths), grids, level counts, code widths,
accumulator widths, element and output types, seeds and counter bases drawn at random, and
code outputs placed at random 16-byte offsets from a 128-byte line.
Codes, sums, payloads and means must be bit-exact; the norm within 1e-6 relative."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import dev, first_diff, gq, host, say

pytestmark = pytest.mark.gpu
U, X = 0, 1
CASES = 40


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def _config(i, K=None, bf16=None):
    rng = np.random.default_rng(90000 + i)
    K = int(rng.choice([1, 2, 3, 4, 5, 8, 11, 16, 23])) if K is None else K
    n = int(rng.integers(1, 40000))
    nseg = int(rng.integers(1, 6))
    cuts = sorted(int(c) // 8 * 8 for c in rng.integers(0, n + 1, nseg - 1))
    off = np.array([0] + cuts + [n], np.int64)
    grid = int(rng.integers(0, 2))
    bits = int(rng.choice([4, 8]))
    maxlv = (1 << (bits - 1)) - 1
    levels = int(rng.integers(1, maxlv + 1)) if grid == U else int(rng.integers(1, min(maxlv, 12) + 1))
    maxlin = levels if grid == U else 1 << (levels - 1)
    acc_bits = 16 if K * maxlin < (1 << 15) and rng.random() < 0.6 else 32
    bf16 = bool(rng.random() < 0.4) if bf16 is None else bf16
    out_dtype = int(rng.random() < 0.3)
    seed = int(rng.integers(0, 1 << 62))
    index_base = int(rng.integers(0, (1 << 32) - n))
    scale_mul = float(10.0 ** rng.uniform(-4, 3))
    xs = []
    for k in range(K):
        x = (rng.standard_normal(n) * scale_mul * 10.0 ** rng.uniform(-1, 1)).astype(np.float32)
        x[rng.random(n) < 0.05] = 0.0
        if bf16:
            x = (x.view(np.uint32) >> 16).astype(np.uint16)
        xs.append(x)
    return dict(K=K, n=n, off=off, grid=grid, bits=bits, levels=levels, acc_bits=acc_bits,
                out_dtype=out_dtype, seed=seed, index_base=index_base, xs=xs)


@pytest.mark.parametrize("i", range(CASES))
def test_random_configuration(orc, i):
    _run(orc, i, _config(i))


@pytest.mark.parametrize("i", range(CASES, CASES + 8))
def test_random_configuration_bf16_16_workers(orc, i):
    """The double-buffered 16-worker bf16 pass (with its fast path) on random lengths, segment
    layouts, grids, levels and seeds."""
    _run(orc, i, _config(i, K=16, bf16=True))


def _run(orc, i, c):
    g = gq()
    K, n, off, grid, bits, levels = c["K"], c["n"], c["off"], c["grid"], c["bits"], c["levels"]
    say("random", i, {k: v for k, v in c.items() if k not in ("xs", "off")}, "nseg", off.size - 1)
    xs = c["xs"]
    xd = [dev(x) for x in xs]
    ref = orc.allreduce_mean(xs, grid, levels, bits, c["acc_bits"], c["seed"], c["index_base"],
                             off, c["out_dtype"])
    S = dev(ref["scale"])
    # global norm
    Sg, _ = g.global_norm(xd, off)
    assert np.all(np.abs(host(Sg).astype(np.float64) - ref["scale"]) <= 1e-6 * ref["scale"])
    # step by step
    codes = [g.quantize_pack(xd[k], S, grid, levels, bits, c["seed"], k, c["index_base"], off)
             for k in range(K)]
    for k in range(K):
        assert np.array_equal(host(codes[k]), ref["codes"][k]), first_diff(host(codes[k]),
                                                                          ref["codes"][k])
    # the same codes written at a random multiple of 16 bytes past a 128-byte line (the
    # quantiser then stores through L2 unless the shift is 0), the bytes around them untouched
    shift = 16 * int(np.random.default_rng(i).integers(0, 8))
    for k in range(K):
        nb = codes[k].numel()
        buf = torch.full((nb + 256,), 0x5A, dtype=torch.uint8, device="cuda")
        base = (-buf.data_ptr()) % 128 + shift
        g.quantize_pack(xd[k], S, grid, levels, bits, c["seed"], k, c["index_base"], off,
                        codes=buf[base:base + nb])
        got = host(buf)
        assert np.array_equal(got[base:base + nb], ref["codes"][k]), (
            shift, first_diff(got[base:base + nb], ref["codes"][k]))
        assert np.all(got[:base] == 0x5A) and np.all(got[base + nb:] == 0x5A)
    sums = g.accumulate_codes(codes, n, grid, levels, bits, c["acc_bits"])
    assert np.array_equal(host(sums), ref["sums"]), first_diff(host(sums), ref["sums"])
    mean = g.dequantize(sums, S, grid, levels, K, c["out_dtype"], off)
    assert np.array_equal(host(mean), ref["mean"]), first_diff(host(mean), ref["mean"])
    # fused, with and without the stored codes and sums
    fused = g.fused_mean(xd, S, grid, levels, bits, c["seed"], c["acc_bits"], c["out_dtype"],
                         c["index_base"], off)
    assert np.array_equal(host(fused), ref["mean"]), first_diff(host(fused), ref["mean"])
    codes2 = [torch.empty_like(cd) for cd in codes]
    sums2 = torch.empty_like(sums)
    g.fused_mean(xd, S, grid, levels, bits, c["seed"], c["acc_bits"], c["out_dtype"],
                 c["index_base"], off, codes=codes2, sums=sums2)
    assert all(torch.equal(a, b) for a, b in zip(codes, codes2)) and torch.equal(sums, sums2)
    # the summable wire payload
    W_ = g.wire_lane_bytes(grid, levels, K)
    if W_:
        pays = [g.quantize_wire(xd[k], S, grid, levels, c["seed"], k, K, c["index_base"], off)
                for k in range(K)]
        prefs = [orc.wire_encode(ref["levels"][k], grid, levels, K) for k in range(K)]
        for k in range(K):
            assert np.array_equal(host(pays[k]), prefs[k]), first_diff(host(pays[k]), prefs[k])
        total = orc.wire_sum(prefs)  # the oracle's own payloads, summed word by word
        wmean = g.dequantize_wire(dev(total), n, S, grid, levels, K, c["out_dtype"], off)
        assert np.array_equal(host(wmean), ref["mean"]), first_diff(host(wmean), ref["mean"])
    # the per-worker-scale baseline on the same inputs
    Sw, _ = orc.worker_scales(xs, int(i % 2), off)
    wref = orc.worker_mean(xs, Sw, grid, levels, c["seed"], c["index_base"], off, c["out_dtype"])
    Swd = dev(np.ascontiguousarray(Sw))
    wgot = g.worker_mean(xd, Swd, grid, levels, c["seed"], c["out_dtype"], c["index_base"], off)
    assert np.array_equal(host(wgot), wref), first_diff(host(wgot), wref)
