"""Per-token RL objective (rlk_rl_token_loss) on the GPU, through the C ABI.

Parity with the fp64 oracle on the same fp32 inputs.  The GPU evaluates in
fp32 with the library's exp (relative error of r a few 2^-24 for the
arguments used), so values and gradients are compared within
    1e-5 * (1 + |r A| + beta (e^d + |d| + 1)) * scale.
Where the clip decision r A <= c A is within 1e-5 (relative) of a tie, fp32
and fp64 may take different branches; both are valid and such tokens are
checked for membership in the two possible answers.  End to end: logp from
the forward, g from the objective, gradients from the backward, against the
oracle's chain on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import selected_token_lm_amd as rlk
import synth
from oracle import rl_loss as orl
from tests.gpu_util import DEV, GRAD_RTOL, dev_inputs, f32_dev, i32_dev, rel_l2, say, to64

pytestmark = pytest.mark.gpu


def token_inputs(T, seed=17):
    gen = np.random.Generator(np.random.PCG64(seed))
    logp = (-gen.uniform(0.0, 15.0, T)).astype(np.float32)
    logp_old = (logp + gen.normal(0, 0.3, T)).astype(np.float32)
    adv = gen.normal(0, 1, T).astype(np.float32)
    ref = (logp + gen.normal(0, 0.2, T)).astype(np.float32)
    y = gen.integers(0, 1000, T).astype(np.int32)
    y[gen.permutation(T)[: T // 10]] = -100
    return logp, logp_old, adv, ref, y


@pytest.mark.parametrize("eps_lo,eps_hi,beta,scale", [(0.2, 0.2, 0.0, 1.0), (0.2, 0.28, 0.04, 1.0 / 4096),
                                                      (0.1, 0.3, 1.0, 2.0)])
def test_matches_oracle(eps_lo, eps_hi, beta, scale):
    T = 100_003
    lp, old, A, ref, y = token_inputs(T)
    say(f"[rl] T={T} eps=({eps_lo},{eps_hi}) beta={beta} scale={scale}")
    loss, g = rlk.rl_token_loss(f32_dev(lp), f32_dev(old), f32_dev(A), i32_dev(y), eps_lo, eps_hi, beta,
                                f32_dev(ref) if beta else None, scale)
    torch.cuda.synchronize()
    loss, g = to64(loss), to64(g)
    ref_loss, ref_g = orl.token_loss(lp, old, A, y, eps_lo, eps_hi, beta, ref if beta else None, scale)
    r = np.exp(lp.astype(np.float64) - old.astype(np.float64))
    d = ref.astype(np.float64) - lp.astype(np.float64)
    mag = np.abs(r * A) + (beta * (np.exp(d) + np.abs(d) + 1) if beta else 0)
    tol = 1e-5 * (1 + mag) * abs(scale)
    c = np.minimum(np.maximum(r, 1 - eps_lo), 1 + eps_hi)
    active = y != -100
    near = active & (np.abs(r * A - c * A) <= 1e-5 * (1 + np.abs(r * A)))
    far = ~near
    say(f"  {int(near.sum())} tokens near a clip boundary; max|dloss|={np.max(np.abs(loss - ref_loss)):.3e}")
    assert np.all(np.abs(loss - ref_loss) <= tol)
    assert np.all(np.abs(g - ref_g)[far] <= tol[far])
    # near a tie: either branch, plus the same KL part
    kl_g = beta * (1 - np.exp(d)) if beta else 0.0
    g_unclipped, g_clipped = (-r * A + kl_g) * scale, kl_g * scale
    ok = (np.abs(g - g_unclipped) <= tol) | (np.abs(g - g_clipped) <= tol)
    assert np.all(ok[near])
    assert np.all(loss[y == -100] == 0) and np.all(g[y == -100] == 0)


def test_bitwise_repeat():
    lp, old, A, ref, y = token_inputs(50_000, seed=23)
    args = (f32_dev(lp), f32_dev(old), f32_dev(A), i32_dev(y), 0.2, 0.28, 0.1, f32_dev(ref), 0.5)
    a = rlk.rl_token_loss(*args)
    b = rlk.rl_token_loss(*args)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_end_to_end_gradients():
    # forward logp -> objective -> g -> backward, against the oracle's chain
    inp = synth.make_inputs(200, 256, 5000, 0.1)
    h, W, y, _ = dev_inputs(inp)
    gen = np.random.Generator(np.random.PCG64(29))
    ref_logp, _ = oracle.forward(inp.h, inp.W, inp.y)
    old = (ref_logp + gen.normal(0, 0.2, inp.T)).astype(np.float32)
    A = gen.normal(0, 1, inp.T).astype(np.float32)
    lref = (ref_logp + gen.normal(0, 0.1, inp.T)).astype(np.float32)
    eps_lo, eps_hi, beta, scale = 0.2, 0.28, 0.05, 1.0 / 180
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    loss, g = rlk.rl_token_loss(logp, f32_dev(old), f32_dev(A), y, eps_lo, eps_hi, beta, f32_dev(lref), scale)
    gh, gW = rlk.linear_logp_bwd(h, W, y, lse, g)
    torch.cuda.synchronize()
    o_loss, o_g = orl.token_loss(ref_logp, old, A, inp.y, eps_lo, eps_hi, beta, lref, scale)
    o_gh, o_gW = oracle.backward(inp.h, inp.W, inp.y, o_g)
    e_h, e_W = rel_l2(to64(gh), o_gh), rel_l2(to64(gW), o_gW)
    say(f"  end to end: loss sum {to64(loss).sum():.6f} vs {o_loss.sum():.6f}; rel L2 grad_h {e_h:.2e} grad_W {e_W:.2e}")
    assert abs(to64(loss).sum() - o_loss.sum()) <= 1e-4 * (1 + abs(o_loss.sum()))
    assert e_h <= GRAD_RTOL and e_W <= GRAD_RTOL


@pytest.mark.parametrize("T,H,V,beta", [(700, 256, 30000, 0.0), (700, 256, 30000, 0.05), (1, 64, 5003, 0.1),
                                        (129, 128, 257, 0.0)])
def test_fused_forward_objective_bitwise_equal_to_separate_calls(T, H, V, beta):
    """rlk_linear_logp_fwd_rl: logp and lse bit-equal to the forward, loss and
    g bit-equal to rlk_rl_token_loss on that logp (the same per-token function
    inside the forward's merge kernel); masked rows 0; an out-of-range target
    gives NaN through both paths."""
    inp = synth.make_inputs(T, H, V, 0.15)
    if T > 5:
        inp.y[5] = V  # out of range: NaN logp, NaN objective
    h, W, y, _ = dev_inputs(inp)
    gen = np.random.Generator(np.random.PCG64(T))
    ref_lp, _ = rlk.linear_logp_fwd(h, W, y)
    old = ref_lp + f32_dev(gen.normal(0, 0.3, T).astype(np.float32))
    adv = f32_dev(gen.normal(0, 1, T).astype(np.float32))
    lref = ref_lp + f32_dev(gen.normal(0, 0.2, T).astype(np.float32)) if beta else None
    say(f"[rl fused] T={T} H={H} V={V} beta={beta}")
    lp, lse, loss, g = rlk.linear_logp_fwd_rl(h, W, y, old, adv, 0.2, 0.28, beta, lref, 1.0 / T)
    ref_lp2, ref_lse = rlk.linear_logp_fwd(h, W, y)
    ref_loss, ref_g = rlk.rl_token_loss(ref_lp2, old, adv, y, 0.2, 0.28, beta, lref, 1.0 / T)
    torch.cuda.synchronize()
    for a, b in ((lp, ref_lp2), (lse, ref_lse), (loss, ref_loss), (g, ref_g)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    masked = torch.from_numpy(inp.y == -100).to(DEV)
    assert torch.all(loss[masked] == 0) and torch.all(g[masked] == 0)
    if T > 5:
        # no silent finite objective for a row without a log-probability
        assert torch.isnan(loss[5]) and torch.isnan(g[5])
