"""The compiler's resource report of the built kernels (CPU only; read from the file the build
writes): no kernel spills registers to scratch memory, and the streaming kernels keep the
occupancy their design relies on to cover HBM latency."""
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RES = os.path.join(ROOT, "allreduce_compatible_gradient_amd", "_build", "kernel_resources.json")


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(RES):
        pytest.skip("the library has not been built here (no resource report)")
    with open(RES) as f:
        return json.load(f)


def test_report_covers_the_kernels(resources):
    names = " ".join(resources)
    for k in ("k_fused", "k_norm_partial", "k_quantize_pack", "k_accumulate", "k_dequantize",
              "k_quantize_wire", "k_worker_mean", "k_decode_workers", "k_lq_ef_mq",
              "k_lq_solve", "k_lq_mtp", "k_lq_qsum", "k_lq_ef_update_q", "k_lq_quant_elems",
              "k_lq_mean_ef", "k_lq_quant_cols", "k_seg_consts"):
        assert k in names, k


def test_no_kernel_spills_to_scratch(resources):
    spills = {k: (v.get("ScratchSize"), v.get("VGPRs Spill")) for k, v in resources.items()
              if v.get("ScratchSize", 0) or v.get("VGPRs Spill", 0)}
    assert not spills, spills


def test_streaming_kernels_keep_four_waves_per_simd(resources):
    """The fused pass without code stores and the per-worker-scale mean fit 128 VGPRs, i.e.
    at least 4 waves per SIMD (the store variants are allowed 2)."""
    low = {}
    for k, v in resources.items():
        streaming = ("k_fused" in k and "Lb0E" in k) or "k_worker_mean" in k \
            or "k_norm_partial" in k
        if streaming and v.get("Occupancy", 0) < 4:
            low[k] = v.get("Occupancy")
    assert not low, low
