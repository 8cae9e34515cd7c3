"""Register, scratch and occupancy budget of every kernel in the last build.

The compiler reports each kernel's resources while building (kernel-resource-
usage remarks, saved by the build next to the objects).  A kernel that spills
to scratch runs several times slower without any numerical symptom, so the
budget is checked here, on the CPU, for every build."""
import json
import os

import pytest

from shared_token_tiled_amd import build as B


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(B.RESOURCES) or os.path.getmtime(B.RESOURCES) < max(
            os.path.getmtime(os.path.join(B.CSRC, f)) for f in os.listdir(B.CSRC)):
        B.build()
    with open(B.RESOURCES) as f:
        return json.load(f)


def test_every_kernel_reported(resources):
    names = " ".join(resources)
    for k in ("k_gemm_mfma", "k_gemm_rows", "k_gemm_f32", "k_attn_bf16", "k_attn_global_bf16", "k_attn_f32",
              "k_qkprep", "k_norm", "k_blend", "k_gather", "k_quant", "k_amax"):
        assert k in names, k


def test_no_scratch_and_no_vgpr_spills(resources):
    bad = {k: v for k, v in resources.items()
           if v.get("scratch_bytes_per_lane", 0) != 0 or v.get("vgpr_spills", 0) != 0}
    assert not bad, bad


def test_lds_fits_the_cu(resources):
    assert all(v.get("lds_bytes", 0) <= 160 * 1024 for v in resources.values())


def test_mfma_kernels_keep_two_waves_per_simd(resources):
    # the 8-wavefront GEMM (128x64 per wavefront) and the attention kernel
    # rely on a second wavefront per SIMD to issue while the other waits
    for k, v in resources.items():
        if ("k_gemm_mfma" in k and k.endswith("Li4EEEvNS_5GemmPE")) or "k_attn_bf16" in k:
            assert v["waves_per_simd"] >= 2, (k, v)
