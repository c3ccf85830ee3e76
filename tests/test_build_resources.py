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


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(B.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [B.HIPCC, *flags, "-DRLK_WAVES=4", "--cuda-device-only", "-c", "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(B.ROOT, "include"),
           os.path.join(B.CSRC, "rlk_api.hip")]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
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
    m = re.match(r"_ZN3rlk(\d+)", mangled)
    n = int(m.group(1))
    return mangled[m.end():m.end() + n]


def test_every_operator_kernel_is_reported(resources):
    names = {short(k) for k in resources}
    assert {"fwd_tiles", "dz_tiles", "grad_tiles", "gemm_tiles", "merge_splits", "merge_parts",
            "dz_saved", "compact_rows", "gather_rows"} <= names, names


def test_no_scratch_in_operator_kernels(resources):
    spills = {k: v["ScratchSize"] for k, v in resources.items()
              if short(k) not in NOT_CHECKED and v.get("ScratchSize", 0) > 0}
    assert not spills, spills


def test_tile_kernels_fit_one_wave_per_simd(resources):
    # the 256 x 256 tile engine holds its accumulators in all 256 AGPRs
    for k, v in resources.items():
        if short(k) in ("fwd_tiles", "dz_tiles", "grad_tiles", "gemm_tiles") and "Li1E" not in k \
                and "Li2E" not in k and "Li3E" not in k:
            assert v["AGPRs"] == 256 and v["VGPRs"] <= 256, (k, v)
