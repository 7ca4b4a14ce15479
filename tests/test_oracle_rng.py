"""Pins of the oracle's counter-based generator (CPU only).

The stochastic rounding draws r = fp32(fmix32(counter XOR key_k)) * 2^-32 -- the 32-bit hash
rounded to the nearest fp32 (ties to even), scaled exactly -- with key_k the low 32 bits of
SplitMix64 output k+1 from the step seed.  Both generators are pinned to published
known-answer values (tests/golden/rng_kat.json); the rounding of the hash is pinned on chosen
hash values (reached through the inverse of the finaliser, tests/draw_helpers.py); the draw is
then checked statistically.
"""
import json
import os

import numpy as np
import pytest

from tests.draw_helpers import counter_for_hash

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rng_kat.json")
M32 = 0xFFFFFFFF


def _rotl(x, r):
    return ((x << r) | (x >> (32 - r))) & M32


def _murmur3_x86_32(data: bytes, seed: int, fmix32) -> int:
    """MurmurHash3_x86_32 body written here; only its finaliser comes from the oracle."""
    c1, c2 = 0xCC9E2D51, 0x1B873593
    h = seed
    nb = len(data) // 4
    for i in range(nb):
        k = int.from_bytes(data[4 * i:4 * i + 4], "little")
        k = _rotl((k * c1) & M32, 15) * c2 & M32
        h = (_rotl(h ^ k, 13) * 5 + 0xE6546B64) & M32
    tail = data[4 * nb:]
    k = 0
    if len(tail) >= 3:
        k ^= tail[2] << 16
    if len(tail) >= 2:
        k ^= tail[1] << 8
    if len(tail) >= 1:
        k ^= tail[0]
        h ^= _rotl((k * c1) & M32, 15) * c2 & M32
    h ^= len(data)
    return fmix32(h)


def test_splitmix64_known_answers(orc):
    kat = json.load(open(GOLDEN))["splitmix64"]
    got = orc.splitmix64_outputs(kat["seed"], len(kat["outputs"]))
    assert got == [int(v) for v in kat["outputs"]]


def test_worker_key_is_splitmix_output(orc):
    kat = json.load(open(GOLDEN))["splitmix64"]
    for k, v in enumerate(kat["outputs"]):
        assert orc.worker_key(kat["seed"], k) == int(v) & M32


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["murmur3_x86_32"])
def test_fmix32_via_murmur3_known_answers(orc, case):
    got = _murmur3_x86_32(case["data"].encode(), case["seed"], orc.fmix32)
    assert got == int(case["hash"], 16)


def _counter_for_hash(orc, key: int, h: int) -> int:
    c = counter_for_hash(key, h)
    assert orc.fmix32(c ^ key) == h
    return c


def test_uniform_is_scaled_nearest_fp32_of_hash(orc):
    key = orc.worker_key(7, 3)
    for c in (0, 1, 12345, M32):
        assert orc.uniform(key, c) == float(np.float32(orc.fmix32(c ^ key))) / 2.0 ** 32


@pytest.mark.parametrize("h,nearest", [
    (0, 0), (1, 1), ((1 << 24) - 1, (1 << 24) - 1),
    ((1 << 24) + 1, 1 << 24),                 # halfway: ties to the even neighbour
    ((1 << 24) + 3, (1 << 24) + 4),           # halfway: ties to the even neighbour
    ((1 << 31) + 127, 1 << 31),               # spacing 256: 127 rounds down
    ((1 << 31) + 129, (1 << 31) + 256),       # 129 rounds up
    ((1 << 31) + 384, (1 << 31) + 512),       # halfway between +256 (odd) and +512 (even)
    (M32 - 127, 1 << 32), (M32, 1 << 32),     # the top hashes round to 2^32: r = 1
])
def test_uniform_rounds_the_hash_to_nearest_even_fp32(orc, h, nearest):
    key = orc.worker_key(11, 2)
    assert orc.uniform(key, _counter_for_hash(orc, key, h)) == nearest / 2.0 ** 32


def test_round_up_compares_the_rounded_hash(orc):
    # s = 1, S = 1, x = 1/2 + 2^-24: u = x, level 0, p = u, p * 2^32 = 2^31 + 256.  The hash
    # 2^31 + 200 is below that threshold but rounds to it (spacing 256), so it does not round
    # up; 2^31 + 100 rounds to 2^31 and does.
    key = orc.worker_key(5, 1)
    x = float(np.float32(0.5 + 2.0 ** -24))
    assert orc.quant_one(0, 1, x, 1.0, key, _counter_for_hash(orc, key, (1 << 31) + 200)) == 0
    assert orc.quant_one(0, 1, x, 1.0, key, _counter_for_hash(orc, key, (1 << 31) + 100)) == 1
    assert orc.quant_one(0, 1, -x, 1.0, key, _counter_for_hash(orc, key, (1 << 31) + 100)) == -1
    # exponential grid, E = 2 (levels 1/2, 1): u = 3/4 + 2^-24 is above 1/2 with
    # p = 1/2 + 2^-23, p * 2^32 = 2^31 + 512; 2^31 + 400 rounds to it, 2^31 + 300 to 2^31 + 256
    x = float(np.float32(0.75 + 2.0 ** -24))
    assert orc.quant_one(1, 2, x, 1.0, key, _counter_for_hash(orc, key, (1 << 31) + 400)) == 1
    assert orc.quant_one(1, 2, x, 1.0, key, _counter_for_hash(orc, key, (1 << 31) + 300)) == 2


def test_zero_draw_at_counter_equal_key(orc):
    # fmix32(0) = 0, so the counter equal to the key draws r = 0 exactly
    key = orc.worker_key(99, 0)
    assert orc.uniform(key, key) == 0.0


def test_hash_uniformity_chi_square(orc):
    from scipy import stats
    h = orc.hash_fill(orc.worker_key(1, 0), 0, 1 << 20)
    counts = np.bincount(h >> 24, minlength=256)
    chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
    assert stats.chi2.sf(chi2, 255) > 1e-4
    # low byte too (the comparison uses all 32 bits)
    counts = np.bincount(h & 0xFF, minlength=256)
    chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
    assert stats.chi2.sf(chi2, 255) > 1e-4


def test_hash_mean_variance_and_worker_independence(orc):
    n = 1 << 20
    r = [orc.hash_fill(orc.worker_key(5, k), 0, n) / 2.0 ** 32 for k in range(4)]
    for x in r:
        assert abs(x.mean() - 0.5) < 5 * np.sqrt(1 / 12 / n)
        assert abs(x.var() - 1 / 12) < 5 * np.sqrt(1 / 180 / n)
    for a in range(4):
        for b in range(a + 1, 4):
            c = np.corrcoef(r[a], r[b])[0, 1]
            assert abs(c) < 5 / np.sqrt(n)
    # consecutive counters of one worker are uncorrelated too
    c = np.corrcoef(r[0][:-1], r[0][1:])[0, 1]
    assert abs(c) < 5 / np.sqrt(n)


def test_distinct_seeds_give_distinct_keys(orc):
    keys = {orc.worker_key(s, k) for s in range(64) for k in range(16)}
    assert len(keys) == 64 * 16
