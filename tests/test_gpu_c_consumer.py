"""The C ABI from plain C: tests/abi/c_consumer (C99, built with gcc by the build step, no
Python or torch in it) calls gq_global_norm, gq_fused_mean, gq_read_status and an invalid call
on the GPU; its results are checked here against the oracle on the same inputs."""
import os
import subprocess

import numpy as np
import pytest

from tests.gpu_helpers import first_diff, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "abi", "c_consumer")
K, N = 3, 10007
OFFSETS = np.array([0, 4096, 4104, N], np.int64)


def _inputs():
    i = np.arange(N, dtype=np.uint64)
    xs = []
    for k in range(K):
        h = (i * 2654435761 + k * 40503) & 0xFFFFFFFF
        xs.append(((h % 2001).astype(np.float32) - np.float32(1000.0)) / np.float32(1000.0))
    return xs


def test_c_program_matches_the_oracle(tmp_path):
    assert os.path.exists(BIN), "tests/abi/c_consumer is not built (run the build step)"
    from oracle import oracle as orc
    say("c consumer")
    xs = _inputs()
    S, _, bad = orc.global_norm(xs, OFFSETS)
    assert not bad
    sin = tmp_path / "scale.bin"
    out = tmp_path / "out.bin"
    S.astype(np.float32).tofile(sin)
    r = subprocess.run([BIN, str(sin), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = out.read_bytes()
    s_gpu = np.frombuffer(raw[:12], np.float32)
    mean = np.frombuffer(raw[12:12 + 4 * N], np.float32)
    status = np.frombuffer(raw[12 + 4 * N:], np.int32)
    assert np.all(np.abs(s_gpu.astype(np.float64) - S) <= 1e-6 * S)
    ref = orc.allreduce_mean(xs, orc.UNIFORM, 31, 8, 16, 99, 5, OFFSETS, scale=S)
    assert np.array_equal(mean, ref["mean"]), first_diff(mean, ref["mean"])
    assert status.tolist() == [0, 1, 1]  # GQ_OK, GQ_EINVAL with a message
