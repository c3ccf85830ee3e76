"""fp64 CPU oracle for the deterministic dense product C = A B^T.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module; the
product path never does, and this module shares no code with it.

"vLLM RL-Kernel v0.1.0: Bitwise Train-Rollout Consistency on ROCm", section
"Implementation on ROCm", lists deterministic MFMA-based GEMM kernels among
the fixes, and section "Boundary Fixes in the RL-Kernel Strict Path" names
what such a GEMM fixes: the K-dimension reduction, the accumulation
precision, the epilogue and the materialization boundary.  What it computes
is the plain definition

    C[i, j] = sum_k A[i, k] * B[j, k]        (A [M, K], B [N, K]: "x W^T")

evaluated here in float64 on the exact values of the bf16 inputs.  Every
bf16 x bf16 product is exact in float64 (8 + 8 significant bits); only the
sum rounds, at float64 precision.

Pins (tests/test_oracle_gemm_pins.py): exact rational brute force on tiny
inputs, the all-ones and identity closed forms, and the non-negative case of
the magnitude bound.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .linear_logp import bf16_to_f64


def _f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def gemm_nt(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C = A B^T in float64 for A [M, K], B [N, K] (bf16 bits or real arrays)."""
    a, b = _f64(A), _f64(B)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("A must be [M, K] and B [N, K]")
    return a @ b.T


def gemm_nt_abs(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """sum_k |A[i, k]| |B[j, k]|: the scale of each element's rounding error."""
    return np.abs(_f64(A)) @ np.abs(_f64(B)).T


def gemm_nt_entries(A: np.ndarray, B: np.ndarray, rows: np.ndarray, cols: np.ndarray):
    """C[rows[n], cols[n]] and its magnitude scale for sampled index pairs,
    one float64 dot product each (for shapes too large to form C)."""
    a, b = _f64(A[rows]), _f64(B[cols])
    return np.einsum("nk,nk->n", a, b), np.einsum("nk,nk->n", np.abs(a), np.abs(b))
