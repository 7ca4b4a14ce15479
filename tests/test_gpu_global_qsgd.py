"""GPU parity of the Global-QSGD path (HIP kernels through the C ABI) against the CPU oracle.

Bar: codes and integer sums bit-exact; decoded means bit-exact too (the decode is one fp32
multiply by a factor both sides compute the same way), which is inside the stated tolerance
of 1e-6 * scale (fp32) and 2e-3 relative (bf16); the global norm within 1e-6 relative.
The oracle's scale is uploaded for the quantiser checks, so a one-ulp difference of the fp64
sum order can never leak into the codes; the GPU's own scale is checked separately.
"""
import numpy as np
import pytest
import torch

from allreduce_compatible_gradient_amd import workloads as W
from tests.gpu_helpers import dev, first_diff, gq, host, say

pytestmark = pytest.mark.gpu

U, X = W.UNIFORM, W.EXP
SEED = 1


def _dt(w):
    return 1 if w.dtype == "bf16" else 0


def _odt(w):
    return 1 if w.out_dtype == "bf16" else 0


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def _oracle_path(orc, w, xs_h, seed=SEED, index_base=0):
    return orc.allreduce_mean(xs_h, w.grid, w.levels, w.bits, w.acc_bits, seed, index_base,
                              w.offsets, _odt(w))


CASES = list(W.GLOBAL_QSGD_WORKLOADS)


@pytest.fixture(scope="module", params=CASES)
def case(request, orc):
    w = W.reduced(request.param)
    say("generate", w.name, "n", w.n, "K", w.K, "nseg", w.nseg)
    xs = W.gradients(w, "cpu")
    xs_h = [W.to_numpy(x) for x in xs]
    ref = _oracle_path(orc, w, xs_h)
    xs_d = [x.to("cuda") for x in xs]
    return w, xs_d, xs_h, ref


def test_global_norm(case):
    w, xs_d, xs_h, ref = case
    say("global_norm", w.name)
    g = gq()
    g.read_status()  # clear a flag left by an earlier test on this context
    norms = torch.empty(w.K * w.nseg, dtype=torch.float64, device="cuda")
    S, _ = g.global_norm(xs_d, w.offsets, norms_out=norms)
    S_h = host(S)
    assert np.all(np.abs(S_h.astype(np.float64) - ref["scale"]) <= 1e-6 * ref["scale"])
    nr = host(norms).reshape(w.K, w.nseg)
    np.testing.assert_allclose(nr, ref["norms"], rtol=1e-12, atol=0)
    assert g.read_status() == g.OK


def test_quantize_pack_bit_exact(case):
    w, xs_d, xs_h, ref = case
    g = gq()
    S = dev(ref["scale"])
    for k in range(w.K):
        say("quantize_pack", w.name, "worker", k)
        codes = g.quantize_pack(xs_d[k], S, w.grid, w.levels, w.bits, SEED, k, 0, w.offsets)
        got = host(codes)
        assert np.array_equal(got, ref["codes"][k]), first_diff(got, ref["codes"][k])


def test_accumulate_bit_exact(case):
    w, xs_d, xs_h, ref = case
    say("accumulate", w.name)
    g = gq()
    codes = [dev(c) for c in ref["codes"]]
    sums = g.accumulate_codes(codes, w.n, w.grid, w.levels, w.bits, w.acc_bits)
    got = host(sums)
    assert ref["overflow"] == 0
    assert np.array_equal(got, ref["sums"]), first_diff(got, ref["sums"])


def test_dequantize_bit_exact(case):
    w, xs_d, xs_h, ref = case
    say("dequantize", w.name)
    g = gq()
    out = g.dequantize(dev(ref["sums"]), dev(ref["scale"]), w.grid, w.levels, w.K, _odt(w),
                       w.offsets)
    got = host(out)
    assert np.array_equal(got, ref["mean"]), first_diff(got, ref["mean"])


def test_fused_bit_exact(case):
    w, xs_d, xs_h, ref = case
    g = gq()
    S = dev(ref["scale"])
    say("fused parity mode", w.name)
    codes = [torch.empty(g.code_bytes(w.n, w.bits), dtype=torch.uint8, device="cuda")
             for _ in range(w.K)]
    sums = torch.empty(w.n, dtype=torch.int16 if w.acc_bits == 16 else torch.int32,
                       device="cuda")
    out = g.fused_mean(xs_d, S, w.grid, w.levels, w.bits, SEED, w.acc_bits, _odt(w),
                       offsets=w.offsets, codes=codes, sums=sums)
    for k in range(w.K):
        assert np.array_equal(host(codes[k]), ref["codes"][k]), first_diff(host(codes[k]),
                                                                          ref["codes"][k])
    assert np.array_equal(host(sums), ref["sums"]), first_diff(host(sums), ref["sums"])
    assert np.array_equal(host(out), ref["mean"]), first_diff(host(out), ref["mean"])
    say("fused fast mode", w.name)
    out2 = g.fused_mean(xs_d, S, w.grid, w.levels, w.bits, SEED, w.acc_bits, _odt(w),
                        offsets=w.offsets)
    assert np.array_equal(host(out2), ref["mean"])


def test_mean_within_stated_tolerance(case):
    """The decoded mean is the exact average of the workers' quantised values up to the output
    rounding (checked against the unrounded decode in fp64): 1e-6 * scale for fp32, half a bf16
    unit in the last place (2^-8 relative) for bf16.  Agreement with the oracle, where the 2e-3
    relative bf16 tolerance applies, is bit-exact (test_fused_bit_exact)."""
    w, xs_d, xs_h, ref = case
    g = gq()
    out = host(g.fused_mean(xs_d, dev(ref["scale"]), w.grid, w.levels, w.bits, SEED, w.acc_bits,
                            _odt(w), offsets=w.offsets))
    if w.out_dtype == "bf16":
        out = (out.astype(np.uint32) << 16).view(np.float32)
    unit = 1.0 / w.levels if w.grid == U else 2.0 ** (1 - w.levels)
    for gi in range(w.nseg):
        lo, hi = w.offsets[gi], w.offsets[gi + 1]
        S = float(ref["scale"][gi])
        exact = ref["sums"][lo:hi].astype(np.float64) * S * unit / w.K
        err = np.abs(out[lo:hi].astype(np.float64) - exact)
        if w.out_dtype == "bf16":
            assert np.all(err <= 2.0 ** -8 * np.abs(exact) * (1 + 1e-6) + 1e-30)
        else:
            assert np.all(err <= 1e-6 * S)


def test_composition_equals_fused_on_gpu_scale(case):
    """GPU norm -> per-worker quantise -> accumulate -> dequantize equals the fused pass, bit
    for bit, and both equal the oracle whenever the GPU scale equals the oracle's."""
    w, xs_d, xs_h, ref = case
    g = gq()
    say("composition", w.name)
    S, _ = g.global_norm(xs_d, w.offsets)
    codes = [g.quantize_pack(xs_d[k], S, w.grid, w.levels, w.bits, SEED, k, 0, w.offsets)
             for k in range(w.K)]
    sums = g.accumulate_codes(codes, w.n, w.grid, w.levels, w.bits, w.acc_bits)
    mean = g.dequantize(sums, S, w.grid, w.levels, w.K, _odt(w), w.offsets)
    fused = g.fused_mean(xs_d, S, w.grid, w.levels, w.bits, SEED, w.acc_bits, _odt(w),
                         offsets=w.offsets)
    assert np.array_equal(host(mean), host(fused))
    if np.array_equal(host(S), ref["scale"]):
        assert np.array_equal(host(mean), ref["mean"])


def test_deterministic(case):
    w, xs_d, xs_h, ref = case
    g = gq()
    a = [host(t) for t in (g.global_norm(xs_d, w.offsets)[0],)]
    b = [host(t) for t in (g.global_norm(xs_d, w.offsets)[0],)]
    assert np.array_equal(a[0], b[0])
