"""Build libgq.so (hipcc, gfx950) in the package directory.

    python -m allreduce_compatible_gradient_amd.build

Every HIP translation unit is compiled with:
  -ffp-contract=off                           one IEEE operation per arithmetic step
  -fhip-fp32-correctly-rounded-divide-sqrt    IEEE fp32 division (inv = s / S)
  -fno-gpu-flush-denormals-to-zero            fp32 denormals preserved
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed-fp32 instructions
and the compiler's per-kernel resource report (registers, scratch, occupancy) is kept in
_build/kernel_resources.json, so that a kernel that starts spilling to scratch is noticed.
"""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["gq_api.cpp", "gq_stream.hip", "gq_lq.hip"]
# measurement probe used by bench.py only (a plain stream of the same memory pattern)
CEILING_SOURCE = "gq_ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libgq_ceiling.so")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-ffp-contract=off",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


RESOURCES = os.path.join(BUILD, "kernel_resources.json")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|VGPRs Spill|SGPRs Spill|"
                     r"LDS Size \[bytes/block\]):\s*(\S+)")


def _resources(stderr: str) -> dict:
    """Per-kernel figures from the -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for key, val in _REMARK.findall(stderr):
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + DEVICE + ["-Rpass-analysis=kernel-resource-usage", "-c",
                                       os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj, _resources(r.stderr)


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        done = list(ex.map(_compile, SOURCES + [CEILING_SOURCE]))
    objs = [o for o, _ in done]
    res = {}
    for _, r in done:
        res.update(r)
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    spills = sorted(k for k, v in res.items()
                    if v.get("ScratchSize", 0) or v.get("VGPRs Spill", 0))
    if spills:
        print("warning: kernels using scratch (register spills): %s" % ", ".join(spills),
              file=sys.stderr)
    _link(objs[-1:], CEILING_LIB)
    _link(objs[:-1], LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
