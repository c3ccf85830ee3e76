"""Build librlk.so (the HIP kernels and the C ABI of include/rlk.h) for gfx950.

    python -m selected_token_lm_amd.build

Compiles in-tree with hipcc; the library lands next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librlk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# rlk_api.hip: the C ABI and every kernel with the RLK_WAVES-wave engine;
# rlk_tiles_w8.hip: the forward, dz and gradient tile kernels with eight waves.
SOURCES = ["rlk_api.hip", "rlk_tiles_w8.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every rounding point is explicit: no a*b+c contraction anywhere
    "-ffp-contract=off",
    "-fno-fast-math",
    # keep fp32 denormals (no flush) in device code
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def build(verbose: bool = True) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    # RLK_WAVES=8: two waves per SIMD in the main unit's engine too (the
    # save-logits forward, the dense product; same results; four is the
    # default)
    waves = os.environ.get("RLK_WAVES", "4")
    if waves not in ("4", "8"):
        raise ValueError(f"RLK_WAVES must be 4 or 8, not {waves!r}")
    cmd = [HIPCC, *FLAGS, f"-DRLK_WAVES={waves}", "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
