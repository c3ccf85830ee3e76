"""Register budget of the hot kernels, checked at build time on the CPU.

Compiles the library's device code with the build's own flags and the
compiler's kernel-resource-usage report, and requires every kernel of the
operator (forward tiles, dz tiles, grad tiles, the dense product, the
merges, the save-logits dz) to use no scratch memory: a spill of the
accumulators or of the epilogue's values to scratch costs memory traffic
on every tile.  (The benchmark-only MFMA ceiling probe is not checked.)
"""
import os
import re
import shutil
import subprocess

import pytest

from selected_token_lm_amd import build as B

NOT_CHECKED = {"mfma_ceiling"}  # benchmark helper (include/rlk_bench.h)


# 16: the default engine (contract 2, v_mfma_f32_16x16x32_bf16); 32: the
# build that still implements contract 1 (v_mfma_f32_32x32x16_bf16)
@pytest.fixture(scope="module", params=[16, 32], ids=["mfma16", "mfma32"])
def resources(request):
    if not os.path.exists(B.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    out = ""
    for src in B.SOURCES:  # both translation units (four- and eight-wave engine)
        cmd = [B.HIPCC, *flags, "-DRLK_WAVES=4", f"-DRLK_MFMA={request.param}", "--cuda-device-only", "-c",
               "-o", os.devnull,
               "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(B.ROOT, "include"),
               os.path.join(B.CSRC, src)]
        out += subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    kern, res = None, {}
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kern = m.group(1)
            res[kern] = {}
            continue
        m = re.search(r"(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and kern:
            res[kern][m.group(1).split()[0]] = int(m.group(2))
    return res


def short(mangled):
    """Kernel name without namespace (rlk:: or rlk::w8::) and signature."""
    m = re.match(r"_ZN3rlk(?:2w8)?(\d+)", mangled)
    n = int(m.group(1))
    return mangled[m.end():m.end() + n]


def test_every_operator_kernel_is_reported(resources):
    names = {short(k) for k in resources}
    assert {"fwd_tiles", "dz_tiles", "grad_tiles", "gemm_tiles", "merge_splits", "merge_parts",
            "dz_saved", "compact_rows", "gather_rows"} <= names, names
    # the eight-wave unit's forward, dz and gradient kernels
    assert {short(k) for k in resources if k.startswith("_ZN3rlk2w8")} == {"fwd_tiles", "dz_tiles",
                                                                          "grad_tiles"}, names


def test_no_scratch_in_operator_kernels(resources):
    spills = {k: v["ScratchSize"] for k, v in resources.items()
              if short(k) not in NOT_CHECKED and v.get("ScratchSize", 0) > 0}
    assert not spills, spills


def test_tile_kernels_register_budget(resources):
    # four waves: the 256 x 256 tile engine holds its accumulators in all 256
    # AGPRs; eight waves (two per SIMD): 128 accumulators per wave, and the
    # whole wave within 256 registers so that two fit a SIMD
    for k, v in resources.items():
        if short(k) not in ("fwd_tiles", "dz_tiles", "grad_tiles", "gemm_tiles"):
            continue
        if k.startswith("_ZN3rlk2w8"):
            assert v["AGPRs"] + v["VGPRs"] <= 256 and v["Occupancy"] >= 2, (k, v)
        elif "Li1E" not in k and "Li2E" not in k and "Li3E" not in k:
            assert v["AGPRs"] == 256 and v["VGPRs"] <= 256, (k, v)
