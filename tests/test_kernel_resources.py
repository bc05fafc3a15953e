"""Register, scratch and LDS use of every kernel in the built library, from
the compiler's resource remarks that the build records
(io_aware_kv_amd/_lib/kernel_resources.json).  A kernel that starts spilling
registers to scratch, or outgrows the LDS its launch assumes, fails here
before any GPU run: such a change once tripled the full-refresh projection
time without changing a single result.
"""
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RES = os.path.join(ROOT, "io_aware_kv_amd", "_lib", "kernel_resources.json")

# the rotating 256 x 256 projection keeps three values in scratch in its
# epilogue (after the K loop); nothing else may spill
# (the E4M3 epilogue of the same kernel keeps 14, the masked E4M3 attention 1)
ALLOWED_SPILL = {"qkv_gemm_kernelILi8ELi2ELi1ELi0E": 3, "qkv_gemm_kernelILi8ELi2ELi1ELi2E": 14,
                 "attn_bf16_kernelILi2ELi2ELb1ELb1E": 1}
LDS_LIMIT = 160 * 1024


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(RES):
        pytest.skip("library not built (python -m io_aware_kv_amd.build)")
    with open(RES) as f:
        return json.load(f)


def test_every_kernel_reported(resources):
    names = " ".join(resources)
    for k in ("qkv_stream2_kernel", "qkv_mid_kernel", "qkv_gemm_kernel", "qkv_bf16_kernel", "attn_bf16_kernel",
              "attn_finish_kernel", "topk_kernel", "map_slots_kernel", "rope_kernel", "cache_write_kernel",
              "conf_partial_kernel", "decide_kernel"):
        assert k in names, k


def test_no_register_spills(resources):
    for name, r in resources.items():
        allowed = next((v for k, v in ALLOWED_SPILL.items() if k in name), 0)
        assert r.get("VGPRs Spill", 0) <= allowed, (name, r)


def test_lds_within_the_compute_unit(resources):
    for name, r in resources.items():
        assert r.get("LDS Size", 0) <= LDS_LIMIT, (name, r)
    # kernels launched two workgroups per compute unit fit twice: every
    # attention instantiation with a two-stage ring (template argument NS = 2,
    # whatever its query-tile rows RT) runs two per compute unit
    two_per_cu = re.compile(r"attn_bf16_kernelILi\d+ELi2E")
    seen = 0
    for name, r in resources.items():
        if two_per_cu.search(name):
            seen += 1
            assert 2 * r["LDS Size"] <= LDS_LIMIT, (name, r)
    assert seen >= 2, "the 64- and 128-row attention kernels were not found"
