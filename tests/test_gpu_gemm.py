"""The deterministic dense product C = A B^T on the GPU, through the C ABI.

Parity: element by element against the fp64 oracle, within the rounding
bound of an fp32 MFMA accumulation chain: K/16 chain steps, each rounding
to fp32 (unit roundoff 2^-24) once or a few times, so
    |C_gpu - C| <= (K/16 + 2) * 2^-22 * sum_k |A[i,k] B[j,k]|
(the factor 4 = 2^-22 / 2^-24 covers a few roundings per step), plus half
a bf16 ulp (2^-9 |C|, taken as 2^-8) when C is stored as bf16.
Self-pins without the oracle: bit-identical repeats, rows of C independent
of the other rows of A and of their order (batch invariance), columns
independent of the other rows of B, and bf16 output = fp32 output rounded
to nearest even.
"""
import numpy as np
import pytest
import torch

import selected_token_lm_amd as rlk
import synth
from oracle import gemm as og
from tests.gpu_util import DEV, bf16_dev, say

pytestmark = pytest.mark.gpu


def operands(M, N, K, seed=11):
    A = synth.normal_bf16(seed, M, K)
    B = synth.normal_bf16(seed + 1, N, K, float(1.0 / np.sqrt(K)))
    return A, B


def bound(K, scale):
    return (K / 16 + 2) * 2.0 ** -22 * scale


def check(C_gpu, A, B, bf16=False):
    C = og.gemm_nt(A, B)
    S = og.gemm_nt_abs(A, B)
    got = C_gpu.float().cpu().numpy().astype(np.float64)
    tol = bound(A.shape[1], S) + (2.0 ** -8 * np.abs(C) if bf16 else 0.0)
    err = np.abs(got - C)
    say(f"  max|dC|={err.max():.3e}, max err/tol={np.max(err / np.maximum(tol, 1e-300)):.3f}")
    assert np.all(err <= tol)


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (64, 256, 256), (300, 260, 128), (513, 770, 320),
                                   (255, 1027, 64), (1030, 513, 1088)])
def test_matches_oracle_fp32(M, N, K):
    say(f"[gemm] M={M} N={N} K={K} fp32")
    A, B = operands(M, N, K)
    C = rlk.gemm_bf16_nt(bf16_dev(A), bf16_dev(B))
    torch.cuda.synchronize()
    assert C.shape == (M, N)
    check(C, A, B)


@pytest.mark.parametrize("M,N,K", [(300, 259, 192), (17, 4099, 256)])
def test_matches_oracle_bf16_and_rounds_once(M, N, K):
    say(f"[gemm] M={M} N={N} K={K} bf16")
    A, B = operands(M, N, K, seed=21)
    Ad, Bd = bf16_dev(A), bf16_dev(B)
    C16 = rlk.gemm_bf16_nt(Ad, Bd, out_dtype=torch.bfloat16)
    C32 = rlk.gemm_bf16_nt(Ad, Bd)
    torch.cuda.synchronize()
    check(C16, A, B, bf16=True)
    # the bf16 result is the fp32 result rounded to nearest even (torch's cast)
    assert torch.equal(C16.contiguous().view(torch.int16), C32.to(torch.bfloat16).view(torch.int16))


def test_bitwise_repeat_and_batch_invariance():
    M, N, K = 700, 600, 512
    say(f"[gemm] invariance M={M} N={N} K={K}")
    A, B = operands(M, N, K, seed=31)
    Ad, Bd = bf16_dev(A), bf16_dev(B)
    full = rlk.gemm_bf16_nt(Ad, Bd)
    again = rlk.gemm_bf16_nt(Ad, Bd)
    assert torch.equal(full, again)
    gen = np.random.Generator(np.random.PCG64(5))
    # rows of C: any subset of A's rows, in any order, alone or with others
    for rows in (np.array([0]), np.array([699]), gen.permutation(M)[:257], gen.permutation(M)):
        sub = rlk.gemm_bf16_nt(Ad[torch.from_numpy(rows).to(DEV)].contiguous(), Bd)
        assert torch.equal(sub, full[torch.from_numpy(rows).to(DEV)])
    # columns of C: any subset of B's rows
    cols = gen.permutation(N)[:301]
    sub = rlk.gemm_bf16_nt(Ad, Bd[torch.from_numpy(cols).to(DEV)].contiguous())
    assert torch.equal(sub, full[:, torch.from_numpy(cols).to(DEV)])
    torch.cuda.synchronize()


def test_lm_head_shape_sampled():
    # the LM-head contraction of the Qwen3-8B-shaped workload (x W^T with
    # H = 4096, V = 151936) at 1000 rows; sampled entries against the oracle
    M, N, K = 1000, 151936, 4096
    say(f"[gemm] LM-head shape M={M} N={N} K={K}, sampled")
    A = synth.normal_bf16(synth.SEED_H, M, K)
    B = synth.normal_bf16(synth.SEED_W, N, K, float(1.0 / np.sqrt(K)))
    C = rlk.gemm_bf16_nt(bf16_dev(A), bf16_dev(B))
    torch.cuda.synchronize()
    gen = np.random.Generator(np.random.PCG64(9))
    rows = gen.integers(0, M, 4096)
    cols = np.concatenate([gen.integers(0, N, 4000), N - 1 - np.arange(96)])
    ref, scale = og.gemm_nt_entries(A, B, rows, cols)
    got = C[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    say(f"  max|dC|={err.max():.3e} over {len(rows)} sampled entries")
    assert np.all(err <= bound(K, scale))


def test_empty_products():
    A = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((5, 64), dtype=torch.bfloat16, device=DEV)
    assert rlk.gemm_bf16_nt(A, B).shape == (0, 5)
    assert rlk.gemm_bf16_nt(B, A).shape == (5, 0)


def test_maximum_k():
    M, N, K = 3, 5, 1 << 20
    say(f"[gemm] max K: M={M} N={N} K={K}")
    A, B = operands(M, N, K, seed=41)
    C = rlk.gemm_bf16_nt(bf16_dev(A), bf16_dev(B))
    torch.cuda.synchronize()
    check(C, A, B)
