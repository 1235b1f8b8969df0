"""The kernels' register, scratch and occupancy budget, as the compiler
reports it for the last default build (``_build/kernel_resources.json``,
written by ``block_diffusion_lm_amd.build``).

Each kernel's tile shape was chosen for a number of resident waves per SIMD
(three workgroups of the D = 128 forward per CU, two dK/dV workgroups per
CU at D = 64, ...).  A source change that adds a few registers can silently
drop a kernel to fewer waves: the forward at D = 96 once went from 168 to
175 VGPRs and lost a third of its occupancy, 9% of its time.  These checks
catch that on the CPU, at build time.  No GPU is involved.
"""
import json
import os

import pytest

from block_diffusion_lm_amd import build as B

# kernel instance -> waves per SIMD it is designed for.  Template arguments:
# fwd_kernel<D, BN, waves, ring, softcap>, bwd_dq_kernel<D, softcap>,
# bwd_dkdv_kernel<D, grouped, softcap>, fwd_fp8_kernel<D>.
WAVES = {
    "fwd_kernel<64,64,4,2,0>": 4, "fwd_kernel<64,64,4,2,1>": 4,
    "fwd_kernel<96,64,4,2,0>": 3, "fwd_kernel<96,64,4,2,1>": 3,
    "fwd_kernel<128,32,4,2,0>": 3, "fwd_kernel<128,32,4,2,1>": 3,
    "fwd_kernel<192,32,4,2,0>": 2, "fwd_kernel<192,32,4,2,1>": 2,
    "fwd_kernel<256,32,4,2,0>": 2, "fwd_kernel<256,32,4,2,1>": 2,
    "bwd_dq_kernel<64,0>": 3, "bwd_dq_kernel<64,1>": 3,
    "bwd_dq_kernel<96,0>": 3, "bwd_dq_kernel<96,1>": 2,
    "bwd_dq_kernel<128,0>": 2, "bwd_dq_kernel<128,1>": 2,
    "bwd_dq_kernel<192,0>": 1, "bwd_dq_kernel<192,1>": 1,
    "bwd_dq_kernel<256,0>": 1, "bwd_dq_kernel<256,1>": 1,
    # two workgroups of 8 waves per CU
    "bwd_dkdv_kernel<64,0,0>": 4, "bwd_dkdv_kernel<64,0,1>": 4,
    "bwd_dkdv_kernel<64,1,0>": 4, "bwd_dkdv_kernel<64,1,1>": 4,
    "bwd_dkdv_kernel<96,0,0>": 4, "bwd_dkdv_kernel<96,1,0>": 4,
    # softcapped D = 96 keeps 64-row tiles at one workgroup per CU
    "bwd_dkdv_kernel<96,0,1>": 2, "bwd_dkdv_kernel<96,1,1>": 2,
    # six pairs (12 waves) per CU; grouped heads keep four pairs
    "bwd_dkdv_kernel<128,0,0>": 3, "bwd_dkdv_kernel<128,0,1>": 3,
    "bwd_dkdv_kernel<128,1,0>": 2, "bwd_dkdv_kernel<128,1,1>": 2,
    "bwd_dkdv_kernel<192,0,0>": 2, "bwd_dkdv_kernel<192,0,1>": 2,
    "bwd_dkdv_kernel<192,1,0>": 2, "bwd_dkdv_kernel<192,1,1>": 2,
    "bwd_dkdv_kernel<256,0,0>": 1, "bwd_dkdv_kernel<256,0,1>": 1,
    "bwd_dkdv_kernel<256,1,0>": 1, "bwd_dkdv_kernel<256,1,1>": 1,
    "fwd_fp8_kernel<64>": 4, "fwd_fp8_kernel<128>": 3,
    "dkdv_reduce_kernel": 8,
}

# Known spills (bytes per lane) that were measured and accepted: the
# softcapped D = 128 forward, held to 168 VGPRs for three waves per SIMD.
SCRATCH_ALLOWED = {"fwd_kernel<128,32,4,2,1>": 8}


def _resources():
    if not os.path.exists(B.RESOURCES):
        pytest.skip("no resource report: run python -m block_diffusion_lm_amd.build first")
    lib = B.LIB
    if os.path.exists(lib) and os.path.getmtime(lib) > os.path.getmtime(B.RESOURCES) + 60:
        pytest.skip("the library was built after the resource report")
    with open(B.RESOURCES) as f:
        return json.load(f)


def test_every_kernel_is_listed():
    res = _resources()
    assert sorted(res) == sorted(WAVES)


@pytest.mark.parametrize("kernel", sorted(WAVES))
def test_occupancy_and_scratch(kernel):
    res = _resources()
    r = res[kernel]
    assert r["waves_per_simd"] >= WAVES[kernel], r
    assert r["scratch"] <= SCRATCH_ALLOWED.get(kernel, 0), r
    # what the CU can hold: 512 registers per lane and SIMD (VGPRs and
    # AGPRs), 160 KiB of LDS
    assert (r["vgprs"] + r["agprs"]) * r["waves_per_simd"] <= 512, r
    assert r["lds"] <= 160 * 1024, r


def test_kernel_key_parsing():
    assert B.kernel_key("_ZN2bd15bwd_dkdv_kernelILi128ELb0ELb1EEEvNS_8AttnArgsEi") == "bwd_dkdv_kernel<128,0,1>"
    assert B.kernel_key("_ZN2bd10fwd_kernelILi96ELi64ELi4ELi2ELb0EEEvNS_8AttnArgsEi") == "fwd_kernel<96,64,4,2,0>"
    assert B.kernel_key("_ZN2bd18dkdv_reduce_kernelEPKfPtS2_xiPKiiiii") == "dkdv_reduce_kernel"
    text = ("x.hip:1:1: remark: Function Name: _ZN2bd14fwd_fp8_kernelILi64EEEvNS_8AttnArgsEi\n"
            "x.hip:1:1: remark:     VGPRs: 101\nx.hip:1:1: remark:     ScratchSize [bytes/lane]: 0\n"
            "x.hip:1:1: remark:     Occupancy [waves/SIMD]: 4\n")
    assert B.parse_resources(text) == {"fwd_fp8_kernel<64>": {"vgprs": 101, "scratch": 0, "waves_per_simd": 4}}
