"""GPU parity of the summable wire payload (gq_quantize_wire / gq_dequantize_wire).

Each worker's payload must equal the oracle's encoding of the oracle's levels byte for byte
(padding included); the K payloads are then added as unsigned 32-bit words with plain torch
integer arithmetic (what an Allreduce-SUM on uint32 does), and the mean decoded from that
sum must equal the oracle's allreduce mean bit for bit.
"""
import numpy as np
import pytest
import torch

from allreduce_compatible_gradient_amd import workloads as W
from tests.gpu_helpers import dev, first_diff, gq, host, say

pytestmark = pytest.mark.gpu
SEED = 5


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def _word_sum(payloads):
    """Word-wise sum mod 2^32 of uint8 payload tensors (torch int64 arithmetic)."""
    acc = torch.zeros(payloads[0].numel() // 4, dtype=torch.int64, device=payloads[0].device)
    for p in payloads:
        acc += p.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    acc &= 0xFFFFFFFF
    acc = torch.where(acc >= 2 ** 31, acc - 2 ** 32, acc).to(torch.int32)
    return acc.view(torch.uint8)


def _check(orc, xs_h, grid, levels, offsets, out_dtype, index_base=0):
    g = gq()
    K = len(xs_h)
    n = xs_h[0].size
    res = orc.allreduce_mean(xs_h, grid, levels, 8, 32, SEED, index_base, offsets, out_dtype)
    S = dev(res["scale"])
    xd = [dev(x) for x in xs_h]
    payloads = []
    for k in range(K):
        p = g.quantize_wire(xd[k], S, grid, levels, SEED, k, K, index_base, offsets)
        want = orc.wire_encode(res["levels"][k], grid, levels, K)
        assert np.array_equal(host(p)[:want.size], want), "worker %d: %s" % (
            k, first_diff(host(p)[:want.size], want))
        payloads.append(p)
    out = g.dequantize_wire(_word_sum(payloads), n, S, grid, levels, K, out_dtype, offsets)
    assert np.array_equal(host(out), res["mean"]), first_diff(host(out), res["mean"])
    return res


@pytest.mark.parametrize("name", W.GLOBAL_QSGD_WORKLOADS)
def test_wire_round_trip_on_the_workloads(orc, name):
    w = W.reduced(name)
    say("wire", w.name, "K", w.K, "lane bytes", gq().wire_lane_bytes(w.grid, w.levels, w.K))
    xs_h = [W.to_numpy(x) for x in W.gradients(w, "cpu")]
    _check(orc, xs_h, w.grid, w.levels, w.offsets, 1 if w.out_dtype == "bf16" else 0)


@pytest.mark.parametrize("grid,levels,K", [(0, 127, 1), (0, 127, 2), (0, 127, 300),
                                           (1, 7, 3), (1, 12, 5), (0, 1, 100)])
@pytest.mark.parametrize("n", [1, 7, 8193, 3 * 8192 + 5])
def test_wire_widths_and_ragged_lengths(orc, grid, levels, K, n):
    """Every lane width (1, 2 and 4 bytes), lengths that leave a partial last word, and
    segments."""
    rng = np.random.default_rng(n + K + levels)
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(K)]
    off = [0, 8, n] if n > 8 else None
    _check(orc, xs, grid, levels, off, 0, index_base=1000)


def test_wire_rejects_widths_that_do_not_fit():
    g = gq()
    assert g.wire_lane_bytes(1, 30, 65536) == 0
    x = torch.zeros(64, device="cuda")
    S = torch.ones(1, device="cuda")
    with pytest.raises(g.GQError) as e:
        g.quantize_wire(x, S, 1, 30, 1, 0, 65536, payload=torch.empty(256, dtype=torch.uint8,
                                                                         device="cuda"))
    assert e.value.code == 1
