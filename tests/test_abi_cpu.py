"""The C ABI without a GPU: the library loads, exports every declared symbol,
and host-side validation rejects bad arguments before touching the device.

Fake pointers below are never dereferenced: each call is built so that a
host check fails (or T == 0) before any HIP call or kernel launch.
"""
import ctypes
import glob
import os
import re

import pytest

import selected_token_lm_amd as rlk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, NULL_ARG, BAD_SHAPE, BAD_ALIGN, UNALIGNED_RANGE, WS_SMALL, HIP, DEVICE, BAD_ARG = range(9)

FAKE = 0x100000      # 16-byte aligned, never dereferenced
MISALIGNED = 0x100008


def declared_functions(headers=None):
    names = set()
    for path in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(rlk_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(rlk.library_path)
    assert [os.path.basename(p) for p in HEADERS] == ["rlk.h", "rlk_bench.h"]
    names = declared_functions()
    # the benchmark helpers live in their own header, apart from the operator's ABI
    bench = declared_functions([os.path.join(ROOT, "include", "rlk_bench.h")])
    assert bench == ["rlk_bench_mfma_ceiling", "rlk_profile_begin", "rlk_profile_end"], bench
    assert len(names) == 18, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(rlk._SIGNATURES)


def test_contract_version_and_status_strings():
    L = rlk.lib()
    # the default build implements contract 2 (16 x 16 x 32 MFMA steps)
    assert L.rlk_contract_version() == 2
    for s in range(9):
        assert len(L.rlk_status_string(s)) > 0
    assert L.rlk_status_string(99) == b"unknown status"


def test_workspace_bytes():
    W = rlk.workspace_bytes
    assert W(0, 4096, 4096, 151936) >= 32 * 38 * 4096 * 8
    assert W(2, 4096, 4096, 151936) == W(0, 4096, 4096, 151936)
    bwd = W(1, 4096, 4096, 151936)
    # the dz block of all 32 splits (4800 padded columns each) fits the default
    # budget; plus the compacted hidden rows
    dz_all = 2 * 4096 * 32 * 4800
    h_act = 2 * 4096 * 4096
    assert dz_all + h_act <= bwd < dz_all + h_act + (1 << 20)
    # at T = 16384 the default budget holds 16 splits (2.5 GiB of dz; a split's
    # dz block is 2 * 16384 * 4800 B), plus the fp32 grad_h accumulator
    bwd3 = W(1, 16384, 2048, 151936)
    assert bwd3 >= 2 * 16384 * 16 * 4800 + 4 * 16384 * 2048
    assert W(0, 0, 64, 10) > 0
    for bad in [(0, -1, 64, 10), (0, 4, 63, 10), (0, 4, 0, 10), (0, 4, 64, 0), (7, 4, 64, 10),
                (0, 4, 64, 8_000_001)]:
        assert W(*bad) == 0, bad


def test_dz_budget_override_is_capped(monkeypatch):
    # RLK_DZ_BUDGET_MB sets the backward's dz block budget up to 3.5 GiB; a
    # larger value acts as 3.5 GiB (tile offsets stay 32-bit)
    W = rlk.workspace_bytes
    shape = (1, 65536, 4096, 151936)  # one split's dz block: 2 * 65536 * 4800 B = 600 MiB
    monkeypatch.setenv("RLK_DZ_BUDGET_MB", "1024")
    one = W(*shape)
    monkeypatch.setenv("RLK_DZ_BUDGET_MB", "2048")
    two = W(*shape)
    monkeypatch.setenv("RLK_DZ_BUDGET_MB", "3584")
    four = W(*shape)
    monkeypatch.setenv("RLK_DZ_BUDGET_MB", "100000")
    big = W(*shape)
    assert one < two < four == big
    per_split = 2 * 65536 * 4800
    assert two - one == per_split and four - two == 2 * per_split  # G = 1 -> 2 -> 4


def fwd(h=FAKE, W=FAKE, y=FAKE, T=64, H=256, V=4096, logp=FAKE, lse=FAKE, ws=FAKE, nbytes=1 << 40):
    return rlk.lib().rlk_linear_logp_fwd(h, W, y, T, H, V, -100, logp, lse, ws, nbytes, None)


def test_fwd_validation():
    assert fwd(h=None) == NULL_ARG
    assert fwd(W=None) == NULL_ARG
    assert fwd(y=None) == NULL_ARG
    assert fwd(logp=None) == NULL_ARG
    assert fwd(ws=None) == NULL_ARG
    assert fwd(T=-1) == BAD_SHAPE
    assert fwd(H=0) == BAD_SHAPE
    assert fwd(H=96) == BAD_SHAPE
    assert fwd(V=0) == BAD_SHAPE
    assert fwd(V=9_000_000) == BAD_SHAPE
    assert fwd(h=MISALIGNED) == BAD_ALIGN
    assert fwd(lse=MISALIGNED) == BAD_ALIGN
    assert fwd(nbytes=100) == WS_SMALL
    assert b"need" in rlk.lib().rlk_last_error_message()
    # T == 0: nothing to do, nothing launched; empty tensors may be NULL
    assert fwd(T=0, nbytes=rlk.workspace_bytes(0, 0, 256, 4096)) == OK
    assert fwd(T=0, h=None, y=None, logp=None, lse=None, ws=None, nbytes=0) == OK
    assert rlk.lib().rlk_last_error_message() == b""
    assert fwd(T=0, H=100) == BAD_SHAPE


def bwd(h=FAKE, W=FAKE, y=FAKE, lse=FAKE, g=FAKE, T=64, H=256, V=4096, gh=FAKE, gW=FAKE, ws=FAKE,
        nbytes=1 << 40):
    return rlk.lib().rlk_linear_logp_bwd(h, W, y, lse, g, T, H, V, -100, gh, gW, ws, nbytes, None)


def test_bwd_validation():
    assert bwd(lse=None) == NULL_ARG
    assert bwd(g=None) == NULL_ARG
    assert bwd(ws=None) == NULL_ARG
    assert bwd(H=100) == BAD_SHAPE
    assert bwd(gW=MISALIGNED) == BAD_ALIGN
    assert bwd(nbytes=1 << 20) == WS_SMALL
    assert bwd(T=0, nbytes=rlk.workspace_bytes(1, 0, 256, 4096)) == OK


def partial(start, length, Vg=151936, T=16, H=64, out=FAKE, nbytes=1 << 40):
    return rlk.lib().rlk_lse_partial(FAKE, FAKE, FAKE, T, H, start, length, Vg, -100, out, FAKE,
                                     nbytes, None)


def test_partial_range_alignment():
    # S = ceil(151936 / 32) = 4748; aligned power-of-two blocks of splits are accepted
    # (checked with T == 0 so nothing is launched)
    for start, length in [(0, 151936), (0, 75968), (75968, 75968), (4748 * 3, 4748),
                          (4748 * 8, 4748 * 8), (4748 * 30, 4748 * 2)]:
        assert partial(start, length, T=0) == OK, (start, length)
    for start, length in [(1, 4748), (0, 4747), (4748, 2 * 4748), (0, 3 * 4748), (75968, 75967),
                          (-4748, 4748), (0, 0), (151936 - 4748, 2 * 4748)]:
        assert partial(start, length) == UNALIGNED_RANGE, (start, length)
    # a vocabulary that is not a multiple of 32: the last block is short
    Vg = 151937  # S = 4749
    assert partial(75984, 151937 - 75984, Vg=Vg, T=0) == OK
    assert partial(75984, 75984, Vg=Vg) == UNALIGNED_RANGE
    assert partial(0, 75968, out=None) == NULL_ARG
    assert partial(0, 75968, nbytes=16) == WS_SMALL


def test_merge_validation():
    L = rlk.lib()
    assert L.rlk_lse_merge(None, 2, FAKE, 8, -100, FAKE, FAKE, None) == NULL_ARG
    assert L.rlk_lse_merge(None, 2, None, 0, -100, None, None, None) == OK
    assert L.rlk_lse_merge(FAKE, 0, FAKE, 8, -100, FAKE, FAKE, None) == BAD_ARG
    assert L.rlk_lse_merge(FAKE, 33, FAKE, 8, -100, FAKE, FAKE, None) == BAD_ARG
    assert L.rlk_lse_merge(FAKE, 2, FAKE, -1, -100, FAKE, FAKE, None) == BAD_SHAPE
    assert L.rlk_lse_merge(MISALIGNED, 2, FAKE, 8, -100, FAKE, FAKE, None) == BAD_ALIGN
    assert L.rlk_lse_merge(FAKE, 2, FAKE, 0, -100, FAKE, FAKE, None) == OK


def gemm(A=FAKE, B=FAKE, M=300, N=260, K=128, C=FAKE, ldc=260, dt=0):
    return rlk.lib().rlk_gemm_bf16_nt(A, B, M, N, K, C, ldc, dt, None)


def test_gemm_validation():
    assert gemm(A=None) == NULL_ARG
    assert gemm(B=None) == NULL_ARG
    assert gemm(C=None) == NULL_ARG
    assert gemm(K=0) == BAD_SHAPE
    assert gemm(K=96) == BAD_SHAPE
    assert gemm(K=1 << 21) == BAD_SHAPE
    assert gemm(M=-1) == BAD_SHAPE
    assert gemm(N=(1 << 24) + 1) == BAD_SHAPE
    assert gemm(ldc=259) == BAD_SHAPE
    assert gemm(ldc=262) == BAD_SHAPE
    assert gemm(dt=2) == BAD_ARG
    assert gemm(A=MISALIGNED) == BAD_ALIGN
    assert gemm(C=MISALIGNED) == BAD_ALIGN
    # empty products launch nothing; their pointers may be NULL
    assert gemm(M=0, A=None, C=None) == OK
    assert gemm(N=0, B=None, C=None) == OK
    assert gemm(M=0, K=96) == BAD_SHAPE


def test_saved_logits_validation():
    L = rlk.lib()
    ld = L.rlk_saved_logits_ld(151936)
    assert ld == 32 * 4800
    assert L.rlk_saved_logits_ld(4096) == 32 * 128
    assert L.rlk_saved_logits_ld(0) == 0
    fs = lambda z=FAKE, ldz=ld, lse=FAKE, T=64: L.rlk_linear_logp_fwd_save(
        FAKE, FAKE, FAKE, T, 4096, 151936, -100, FAKE, lse, z, ldz, FAKE, 1 << 40, None)
    assert fs(z=None) == NULL_ARG
    assert fs(lse=None) == NULL_ARG
    assert fs(ldz=ld - 4) == BAD_SHAPE
    assert fs(ldz=ld + 2) == BAD_SHAPE
    assert fs(z=MISALIGNED) == BAD_ALIGN
    assert fs(T=0, z=None) == OK
    bs = lambda z=FAKE, ldz=ld, T=64: L.rlk_linear_logp_bwd_saved(
        FAKE, FAKE, FAKE, FAKE, FAKE, z, ldz, T, 4096, 151936, -100, FAKE, FAKE, FAKE, 1 << 40, None)
    assert bs(z=None) == NULL_ARG
    assert bs(ldz=100) == BAD_SHAPE
    assert bs(z=MISALIGNED) == BAD_ALIGN
    assert bs(T=0, z=None, ldz=0) == OK


def test_rl_loss_validation():
    L = rlk.lib()
    f = lambda T=8, elo=0.2, ehi=0.2, beta=0.0, ref=None, lp=FAKE: L.rlk_rl_token_loss(
        lp, FAKE, FAKE, ref, FAKE, T, -100, elo, ehi, beta, 1.0, FAKE, FAKE, None)
    assert f(lp=None) == NULL_ARG
    assert f(beta=0.1) == NULL_ARG          # beta > 0 needs logp_ref
    assert f(elo=1.0) == BAD_ARG
    assert f(elo=-0.1) == BAD_ARG
    assert f(beta=-1.0) == BAD_ARG
    assert f(T=-1) == BAD_SHAPE
    assert f(T=0, lp=None) == OK


def test_binding_refuses_host_tensors():
    import torch
    h = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        rlk.linear_logp_fwd(h, h, torch.zeros(4, dtype=torch.int32))


def test_noalloc_validation():
    L = rlk.lib()

    def call(T=64, H=256, V=4096, h=FAKE, logp=FAKE, lse=FAKE):
        return L.rlk_linear_logp_fwd_noalloc(h, FAKE, FAKE, T, H, V, -100, logp, lse, None)

    assert rlk.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert call(logp=None) == NULL_ARG
    assert call(H=96) == BAD_SHAPE
    assert call(lse=MISALIGNED) == BAD_ALIGN
    assert call(T=0, h=None, logp=None, lse=None) == OK
    # more workspace than the fixed scratch holds: refused on the host
    assert rlk.workspace_bytes(0, 4096, 4096, 151936) > rlk.NOALLOC_SCRATCH_BYTES
    assert call(T=4096, H=4096, V=151936) == WS_SMALL
    assert b"fixed device scratch" in L.rlk_last_error_message()


def test_fused_rl_forward_validation():
    L = rlk.lib()

    def call(T=64, H=256, V=4096, old=FAKE, adv=FAKE, ref=None, eps_lo=0.2, beta=0.0, logp=FAKE, loss=FAKE,
             g=FAKE, nbytes=1 << 40):
        return L.rlk_linear_logp_fwd_rl(FAKE, FAKE, FAKE, T, H, V, -100, old, adv, ref, eps_lo, 0.2, beta, 1.0,
                                        logp, FAKE, loss, g, FAKE, nbytes, None)

    assert call(old=None) == NULL_ARG
    assert call(adv=None) == NULL_ARG
    assert call(beta=0.1) == NULL_ARG          # logp_ref is required with a KL term
    assert call(eps_lo=1.0) == BAD_ARG
    assert call(beta=-1.0) == BAD_ARG
    assert call(loss=None, g=None) == NULL_ARG
    assert call(H=96) == BAD_SHAPE
    assert call(nbytes=10) == WS_SMALL
    assert call(T=0, old=None, adv=None, logp=None, loss=None, g=None) == OK


def test_mfma_ceiling_validation():
    # the benchmark helper checks its arguments before any device call
    L = rlk.lib()
    f = L.rlk_bench_mfma_ceiling
    assert f(FAKE, FAKE, 0, 10, None) == BAD_ARG
    assert f(FAKE, FAKE, 65537, 10, None) == BAD_ARG
    assert f(FAKE, FAKE, 256, 0, None) == BAD_ARG
    assert f(None, FAKE, 256, 10, None) == NULL_ARG
    assert f(FAKE, None, 256, 10, None) == NULL_ARG
    assert f(MISALIGNED, FAKE, 256, 10, None) == BAD_ALIGN
