"""Backward (grad_h, grad_W) on the GPU, through the C ABI.

Parity: relative L2 <= 2e-2 against the fp64 oracle on whole tensors (the
full Qwen3 shapes, every element and every tile, are in
test_gpu_full_size.py).
Self-pins: bit-identical repeats, grad_h rows independent of batch mates,
inactive rows exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
import selected_token_lm_amd as rlk
import synth
from tests.gpu_util import DEV, GRAD_RTOL, config, dev_inputs, rel_l2, say, target_sweep, to64

pytestmark = pytest.mark.gpu


def fwd_bwd(inp):
    h, W, y, g = dev_inputs(inp)
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    gh, gW = rlk.linear_logp_bwd(h, W, y, lse, g)
    torch.cuda.synchronize()
    return (h, W, y, g), logp, lse, gh, gW


@pytest.mark.parametrize("T,H,V,mask", [
    (192, 256, 5000, 0.15),
    (300, 192, 20000, 0.15),
    (64, 64, 100, 0.0),      # tiny vocabulary: 25 non-empty splits of 4 columns
    (129, 128, 4096, 0.3),
])
def test_small_shapes_match_oracle(T, H, V, mask):
    say(f"bwd T={T} H={H} V={V}")
    inp = synth.make_inputs(T, H, V, mask)
    _, logp, lse, gh, gW = fwd_bwd(inp)
    ref_gh, ref_gW = oracle.backward(inp.h, inp.W, inp.y, inp.g)
    e_h = rel_l2(to64(gh), ref_gh)
    e_W = rel_l2(to64(gW), ref_gW)
    say(f"  relL2 grad_h={e_h:.3e} grad_W={e_W:.3e}")
    assert e_h <= GRAD_RTOL and e_W <= GRAD_RTOL
    masked = inp.y == -100
    assert torch.all(gh[torch.from_numpy(masked).to(DEV)] == 0)


def test_target_at_every_tile_position():
    """The delta term of dz lands on the target column at any of a tile's
    lane / element positions and at the split and vocabulary edges."""
    inp = target_sweep()
    say(f"bwd target sweep T={inp.T} H={inp.H} V={inp.V}")
    _, logp, lse, gh, gW = fwd_bwd(inp)
    ref_gh, ref_gW = oracle.backward(inp.h, inp.W, inp.y, inp.g)
    e_h = rel_l2(to64(gh), ref_gh)
    e_W = rel_l2(to64(gW), ref_gW)
    # the target columns' rows of grad_W carry the delta terms: each on its own
    act = inp.y[inp.y >= 0]
    e_Wy = rel_l2(to64(gW)[act], ref_gW[act])
    say(f"  relL2 grad_h={e_h:.3e} grad_W={e_W:.3e} target rows of grad_W={e_Wy:.3e}")
    assert e_h <= GRAD_RTOL and e_W <= GRAD_RTOL and e_Wy <= GRAD_RTOL


def test_grad_subsets_and_flags():
    inp = synth.make_inputs(200, 128, 3000, 0.15)
    (h, W, y, g), logp, lse, gh, gW = fwd_bwd(inp)
    gh_only, none_W = rlk.linear_logp_bwd(h, W, y, lse, g, need_grad_W=False)
    none_h, gW_only = rlk.linear_logp_bwd(h, W, y, lse, g, need_grad_h=False)
    assert none_W is None and none_h is None
    assert torch.equal(gh_only, gh) and torch.equal(gW_only, gW)


def test_all_rows_masked_gives_zero_gradients():
    inp = synth.make_inputs(100, 64, 700, 0.0)
    inp.y[:] = -100
    _, logp, lse, gh, gW = fwd_bwd(inp)
    assert torch.all(gh == 0) and torch.all(gW == 0)


def test_bitwise_repeat():
    inp = synth.make_inputs(400, 256, 25000, 0.15)
    (h, W, y, g), logp, lse, gh, gW = fwd_bwd(inp)
    for _ in range(3):
        gh2, gW2 = rlk.linear_logp_bwd(h, W, y, lse, g)
        assert torch.equal(gh, gh2) and torch.equal(gW, gW2)


def test_grad_h_rows_independent_of_batch():
    inp = synth.make_inputs(600, 128, 9000, 0.15)
    (h, W, y, g), logp, lse, gh, gW = fwd_bwd(inp)
    for rows in synth.rebatch_plan(600, sizes=(1, 7, 128, 500)):
        r = torch.from_numpy(rows).to(DEV)
        gh_r, _ = rlk.linear_logp_bwd(h[r], W, y[r], lse[r], g[r], need_grad_W=False)
        assert torch.equal(gh_r, gh[r]), len(rows)


def test_autograd_wrapper():
    inp = synth.make_inputs(64, 128, 2000, 0.1)
    h, W, y, g = dev_inputs(inp)
    h.requires_grad_(True)
    W.requires_grad_(True)
    logp = rlk.linear_logp(h, W, y)
    (logp * g).sum().backward()
    ref_gh, ref_gW = oracle.backward(inp.h, inp.W, inp.y, inp.g)
    assert rel_l2(to64(h.grad), ref_gh) <= GRAD_RTOL
    assert rel_l2(to64(W.grad), ref_gW) <= GRAD_RTOL


# (the full Qwen3-shaped parity cases, every element, are in test_gpu_full_size.py)


def test_split_grouping_changes_no_bit(monkeypatch):
    # the backward processes the vocabulary in groups of splits sized by a
    # workspace budget; any grouping must give the same bits
    inp = synth.make_inputs(700, 256, 30000, 0.15)
    (h, W, y, g), logp, lse, gh, gW = fwd_bwd(inp)
    for mb in ("1", "4", "16"):
        monkeypatch.setenv("RLK_DZ_BUDGET_MB", mb)
        gh2, gW2 = rlk.linear_logp_bwd(h, W, y, lse, g)
        torch.cuda.synchronize()
        assert torch.equal(gh, gh2) and torch.equal(gW, gW2), mb


@pytest.mark.parametrize("T,H,V,budget_mb", [
    (700, 256, 30000, None),    # one group of splits
    (700, 256, 30000, "4"),     # several groups: the chain continues through the fp32 accumulator
    (300, 512, 20000, None),    # ragged rows and a ragged last column tile of H
])
def test_grad_h_row_passes_change_no_bit(monkeypatch, T, H, V, budget_mb):
    # grad_h tiles computed whole or in 32-row passes: the same MFMA chain
    # per element, so the same bits
    if budget_mb:
        monkeypatch.setenv("RLK_DZ_BUDGET_MB", budget_mb)
    inp = synth.make_inputs(T, H, V, 0.15)
    h, W, y, g = dev_inputs(inp)
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    out = {}
    for passes in ("0", "1"):
        monkeypatch.setenv("RLK_GRAD_H_PASSES", passes)
        out[passes] = rlk.linear_logp_bwd(h, W, y, lse, g)
        torch.cuda.synchronize()
    say(f"  row passes T={T} H={H} V={V} budget={budget_mb}")
    assert torch.equal(out["0"][0], out["1"][0]) and torch.equal(out["0"][1], out["1"][1])
    ref_gh, _ = oracle.backward(inp.h, inp.W, inp.y, inp.g)
    assert rel_l2(to64(out["1"][0]), ref_gh) <= GRAD_RTOL


@pytest.mark.parametrize("T,H,V", [(3, 65536, 600), (5, 64, 8_000_000)])
def test_maximum_hidden_and_vocabulary(T, H, V):
    say(f"bwd max sizes T={T} H={H} V={V}")
    inp = synth.make_inputs(T, H, V, 0.0)
    _, logp, lse, gh, gW = fwd_bwd(inp)
    ref_gh, ref_gW = oracle.backward(inp.h, inp.W, inp.y, inp.g)
    e_h = rel_l2(to64(gh), ref_gh)
    e_W = rel_l2(to64(gW), ref_gW)
    say(f"  relL2 grad_h={e_h:.3e} grad_W={e_W:.3e}")
    assert e_h <= GRAD_RTOL and e_W <= GRAD_RTOL


def test_out_of_range_target_poisons_gradients():
    # a target outside [0, V) has no log-probability (the forward writes NaN);
    # the backward must not return finite, silently wrong gradients for it
    inp = synth.make_inputs(40, 64, 700, 0.1)
    inp.y[5] = 700
    (h, W, y, g), logp, lse, gh, gW = fwd_bwd(inp)
    assert torch.isnan(logp[5])
    assert torch.all(torch.isnan(gh[5]))
    others = torch.ones(inp.T, dtype=torch.bool, device=DEV)
    others[5] = False
    assert torch.all(torch.isfinite(gh[others]))
    assert torch.all(torch.isnan(gW))
