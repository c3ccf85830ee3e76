"""Pins of the fp64 GEMM oracle (oracle/gemm.py) to things other than itself.

P-G1 exact rational arithmetic on tiny bf16 inputs (pure-Python brute force);
P-G2 closed forms: all-ones operands give K everywhere; an identity A gives B^T;
P-G3 the magnitude scale equals C for non-negative operands and bounds |C|;
P-G4 the sampled-entry form agrees with the exact brute force.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import gemm as og

ONE_BF16 = 0x3F80  # 1.0 in bf16


def _exact(bits: np.ndarray):
    """bf16 bits -> exact Fractions, decoded from sign / exponent / mantissa."""
    out = []
    for row in np.asarray(bits, dtype=np.uint16):
        r = []
        for u in row:
            u = int(u)
            sign = -1 if u >> 15 else 1
            e = (u >> 7) & 0xFF
            m = u & 0x7F
            assert 0 < e < 255, "normal numbers only"
            r.append(sign * Fraction(128 + m, 128) * Fraction(2) ** (e - 127))
        out.append(r)
    return out


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (6, 4, 16), (1, 9, 33)])
def test_exact_brute_force(M, N, K):
    A = synth.normal_bf16(101, M, K)
    B = synth.normal_bf16(102, N, K, 0.5)
    a, b = _exact(A), _exact(B)
    C = og.gemm_nt(A, B)
    for i in range(M):
        for j in range(N):
            ref = sum(a[i][k] * b[j][k] for k in range(K))
            scale = float(sum(abs(a[i][k] * b[j][k]) for k in range(K)))
            assert abs(C[i, j] - float(ref)) <= 2.0 ** -50 * scale, (i, j)


def test_all_ones_closed_form():
    M, N, K = 4, 3, 640
    A = np.full((M, K), ONE_BF16, dtype=np.uint16)
    B = np.full((N, K), ONE_BF16, dtype=np.uint16)
    assert np.array_equal(og.gemm_nt(A, B), np.full((M, N), float(K)))


def test_identity_closed_form():
    K, N = 8, 5
    A = np.zeros((K, K), dtype=np.uint16)
    A[np.arange(K), np.arange(K)] = ONE_BF16
    B = synth.normal_bf16(103, N, K)
    assert np.array_equal(og.gemm_nt(A, B), synth.bf16_bits_to_f32(B).astype(np.float64).T)


def test_magnitude_scale():
    A = synth.normal_bf16(104, 5, 64)
    B = synth.normal_bf16(105, 6, 64)
    pos_a = A & np.uint16(0x7FFF)  # clear the sign bits: |A|
    pos_b = B & np.uint16(0x7FFF)
    assert np.array_equal(og.gemm_nt_abs(A, B), og.gemm_nt(pos_a, pos_b))
    assert np.all(np.abs(og.gemm_nt(A, B)) <= og.gemm_nt_abs(A, B))


def test_sampled_entries_match_brute_force():
    A = synth.normal_bf16(106, 7, 24)
    B = synth.normal_bf16(107, 9, 24)
    a, b = _exact(A), _exact(B)
    rows = np.array([0, 6, 3, 3])
    cols = np.array([8, 0, 4, 4])
    vals, scale = og.gemm_nt_entries(A, B, rows, cols)
    for n, (i, j) in enumerate(zip(rows, cols)):
        ref = sum(a[i][k] * b[j][k] for k in range(24))
        assert abs(vals[n] - float(ref)) <= 2.0 ** -50 * scale[n]
