"""Save-logits variant (rlk_linear_logp_fwd_save / rlk_linear_logp_bwd_saved).

The saved logits are the fp32 values the chunk statistics come from, so the
variant must reproduce the default path bit for bit: logp and lse of the
forward, grad_h and grad_W of the backward.  The saved logits themselves
are compared with the fp64 oracle's h W^T within the rounding bound of an
fp32 MFMA chain, (H/16 + 2) * 2^-22 * sum_k |h_k W_vk| (the same bound as the
dense-product tests).
"""
import numpy as np
import pytest
import torch

import selected_token_lm_amd as rlk
import synth
from oracle import gemm as og
from tests.gpu_util import DEV, bf16_dev, config, dev_inputs, say, target_sweep

pytestmark = pytest.mark.gpu


def vocab_of_saved(V):
    """(split-layout column -> vocabulary index, valid mask) of a saved row."""
    S = -(-V // 32)
    S_pad = -(-S // 64) * 64
    col = np.arange(32 * S_pad)
    s, c = col // S_pad, col % S_pad
    v = s * S + c
    valid = (c < S) & (v < V)
    return v, valid


def check_saved_logits(inp, z, rows):
    v, valid = vocab_of_saved(inp.V)
    cols = np.nonzero(valid)[0]
    got = z[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].cpu().numpy().astype(np.float64)
    ref = og.gemm_nt(inp.h[rows], inp.W[v[cols]])
    scale = og.gemm_nt_abs(inp.h[rows], inp.W[v[cols]])
    err = np.abs(got - ref)
    tol = (inp.H / 16 + 2) * 2.0 ** -22 * scale
    say(f"  saved logits: max|dz|={err.max():.3e} over {err.size} entries")
    assert np.all(err <= tol)


def same_bits(a, b):
    """Bit-identical tensors (fp32 or bf16)."""
    iv = torch.int32 if a.dtype == torch.float32 else torch.int16
    return a.dtype == b.dtype and torch.equal(a.view(iv), b.view(iv))


@pytest.mark.parametrize("T,H,V,mask", [(64, 256, 4096, 0.0), (300, 192, 5000, 0.2), (37, 64, 1000, 0.3)])
def test_small_shapes_bitwise_equal_to_recompute(T, H, V, mask):
    say(f"[saved] T={T} H={H} V={V} mask={mask}")
    check_equal_to_recompute(synth.make_inputs(T, H, V, mask))


def test_target_sweep_bitwise_equal_to_recompute():
    inp = target_sweep()
    say(f"[saved] target sweep T={inp.T} H={inp.H} V={inp.V}")
    check_equal_to_recompute(inp)


def check_equal_to_recompute(inp):
    h, W, y, g = dev_inputs(inp)
    logp0, lse0 = rlk.linear_logp_fwd(h, W, y)
    logp1, lse1, z = rlk.linear_logp_fwd_save(h, W, y)
    gh0, gW0 = rlk.linear_logp_bwd(h, W, y, lse0, g)
    gh1, gW1 = rlk.linear_logp_bwd_saved(h, W, y, lse1, g, z)
    torch.cuda.synchronize()
    assert same_bits(logp0, logp1) and same_bits(lse0, lse1)
    assert same_bits(gh0, gh1) and same_bits(gW0, gW1)
    act = np.nonzero(inp.y != -100)[0]
    check_saved_logits(inp, z, act)


def test_grad_subsets():
    inp = synth.make_inputs(100, 128, 3000, 0.1)
    h, W, y, g = dev_inputs(inp)
    _, lse, z = rlk.linear_logp_fwd_save(h, W, y)
    gh_full, gW_full = rlk.linear_logp_bwd_saved(h, W, y, lse, g, z)
    gh, gW = rlk.linear_logp_bwd_saved(h, W, y, lse, g, z, need_grad_W=False)
    assert gW is None and same_bits(gh, gh_full)
    gh, gW = rlk.linear_logp_bwd_saved(h, W, y, lse, g, z, need_grad_h=False)
    assert gh is None and same_bits(gW, gW_full)
    torch.cuda.synchronize()


def test_qwen3_8b_shape_bitwise_equal_to_recompute():
    inp = config("qwen3_8b")
    say(f"[saved] Qwen3-8B shape T={inp.T} H={inp.H} V={inp.V}")
    h, W, y, g = dev_inputs(inp)
    logp0, lse0 = rlk.linear_logp_fwd(h, W, y)
    logp1, lse1, z = rlk.linear_logp_fwd_save(h, W, y)
    assert same_bits(logp0, logp1) and same_bits(lse0, lse1)
    gh0, gW0 = rlk.linear_logp_bwd(h, W, y, lse0, g)
    gh1, gW1 = rlk.linear_logp_bwd_saved(h, W, y, lse1, g, z)
    torch.cuda.synchronize()
    assert same_bits(gh0, gh1)
    assert same_bits(gW0, gW1)
    del gW0, gW1
    # sampled saved logits against fp64 dot products
    gen = np.random.Generator(np.random.PCG64(13))
    act = np.nonzero(inp.y != -100)[0]
    rows = gen.choice(act, 2048)
    v_of, valid = vocab_of_saved(inp.V)
    cols = gen.choice(np.nonzero(valid)[0], 2048)
    ref, scale = og.gemm_nt_entries(inp.h, inp.W, rows, v_of[cols])
    got = z[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    say(f"  sampled saved logits: max|dz|={err.max():.3e}")
    assert np.all(err <= (inp.H / 16 + 2) * 2.0 ** -22 * scale)
