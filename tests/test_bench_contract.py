"""bench.py's host-side contract (CPU only; nothing here touches a GPU): runs on more than one
GPU are refused with a message, the counter traffic is reported only for the kernel source it
was measured on, and the CPU baseline leg times the oracle and describes its sample."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_follows_the_kernel_source(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: t["kernel_source_sha256_16"])
    assert bench.measured_traffic(1) == t["hbm_bytes_per_launch"]
    # the counters' bytes per launch are the fused pass's algorithmic bytes to 0.01%
    assert abs(t["hbm_bytes_per_launch"] / 46.8e9 - 1) < 1e-4
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic(1) is None


def test_cpu_baseline_times_the_oracle_on_a_sample():
    sys.path.insert(0, ROOT)
    import bench
    from allreduce_compatible_gradient_amd import workloads as W
    w = W.get("flat-1.3G-f32-K8-uniform127", n=1 << 14)
    grads = W.gradients(w, "cpu")
    cb = bench.cpu_baseline(grads, w, 1 << 12)
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["unit"] == "GB/s"
    assert cb["value"] > 0 and str(1 << 12) in cb["sample"]
