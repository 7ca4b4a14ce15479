"""The C ABI from plain C: tests/abi/c_consumer (C99, built with gcc by the build step, no
Python or torch in it) calls gq_global_norm, gq_fused_mean, gq_read_status, an invalid call,
gq_quantize_pack for every worker with gq_accumulate_codes and gq_dequantize, and one
gq_powersgd_logquant step on the GPU.  The Global-QSGD results are checked against the oracle
on the same inputs, the LQ-SGD step against the same call made through the Python binding on
the same inputs (bit for bit: one library, one arithmetic)."""
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
LN, LM, LR = 96, 72, 3


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
    pos = [0]

    def take(count, dtype):
        a = np.frombuffer(raw, dtype, count, pos[0])
        pos[0] += a.nbytes
        return a
    s_gpu = take(3, np.float32)
    mean = take(N, np.float32)
    status = take(3, np.int32)
    mean2 = take(N, np.float32)
    pc, pm = take(LN * LR, np.int8), take(LR, np.float32)
    qc, qm = take(LM * LR, np.int8), take(LR, np.float32)
    e_after, q_after = take(LN * LM, np.float32), take(LM * LR, np.float32)
    assert pos[0] == len(raw)
    assert np.all(np.abs(s_gpu.astype(np.float64) - S) <= 1e-6 * S)
    ref = orc.allreduce_mean(xs, orc.UNIFORM, 31, 8, 16, 99, 5, OFFSETS, scale=S)
    assert np.array_equal(mean, ref["mean"]), first_diff(mean, ref["mean"])
    assert status.tolist() == [0, 1, 1]  # GQ_OK, GQ_EINVAL with a message
    assert np.array_equal(mean2, ref["mean"]), first_diff(mean2, ref["mean"])

    # the LQ-SGD step through the Python binding on the same inputs
    import torch
    from tests.gpu_helpers import gq
    t = np.arange(LN * LM, dtype=np.uint64)
    h = (t * 2654435761 + 12345) & 0xFFFFFFFF
    G = ((h % 2001).astype(np.float32) - np.float32(1000)) / np.float32(1000) * np.float32(0.001)
    u = np.arange(LM * LR, dtype=np.uint64)
    h = (u * 40503 + 777) & 0xFFFFFFFF
    Q = ((h % 2001).astype(np.float32) - np.float32(1000)) / np.float32(1000)
    Gd = torch.from_numpy(G.reshape(LN, LM)).cuda()
    Ed = torch.zeros_like(Gd)
    Qd = torch.from_numpy(Q.reshape(LM, LR).copy()).cuda()
    o = gq().powersgd_logquant(Gd, Ed, Qd, 10.0, 8, bits_q=6, want_hat=False)
    for what, got, want in (("p_codes", pc, o["p_codes"]), ("p_colmax", pm, o["p_colmax"]),
                            ("q_codes", qc, o["q_codes"]), ("q_colmax", qm, o["q_colmax"]),
                            ("E", e_after, Ed), ("Q", q_after, Qd)):
        want = want.cpu().numpy().reshape(-1)
        assert np.array_equal(got, want), "%s: %s" % (what, first_diff(got, want))
    assert np.any(pc != 0) and np.any(qc != 0) and np.abs(qc).max() <= 31
