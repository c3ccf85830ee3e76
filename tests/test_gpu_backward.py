"""Backward (grad_h, grad_W) on the GPU, through the C ABI.

Parity: relative L2 <= 2e-2 against the fp64 oracle (whole tensors at small
sizes; sampled rows of grad_h and sampled vocabulary rows of grad_W at the
full Qwen3 shapes, where the oracle evaluates those entries one by one).
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


# --- full shapes -------------------------------------------------------------------

def _full_shape_check(name, n_rows=16, n_vocab=24):
    inp = config(name)
    say(f"{name}: fwd+bwd on the GPU")
    (h, W, y, g), logp, lse, gh, gW = fwd_bwd(inp)
    rng = np.random.Generator(np.random.PCG64(5))
    act = np.nonzero(inp.y != -100)[0]
    rows = rng.choice(act, n_rows, replace=False)
    say(f"  oracle grad_h on {n_rows} rows")
    ref_rows = oracle.backward_rows(inp.h, inp.W, inp.y, inp.g, rows)
    e_h = rel_l2(to64(gh[torch.from_numpy(rows).to(DEV)]), ref_rows)
    say(f"  relL2 grad_h(sampled rows) = {e_h:.3e}")
    assert e_h <= GRAD_RTOL
    vr = np.concatenate([rng.choice(inp.V, n_vocab - 4, replace=False), inp.y[rows[:4]]])
    say(f"  oracle grad_W on {len(vr)} vocabulary rows (full log-sum-exp first)")
    ref_W = oracle.grad_W_rows(inp.h, inp.W, inp.y, inp.g, vr)
    e_W = rel_l2(to64(gW[torch.from_numpy(vr).to(DEV)]), ref_W)
    say(f"  relL2 grad_W(sampled rows) = {e_W:.3e}")
    assert e_W <= GRAD_RTOL
    # property at any size: every column of grad_W sums to ~0 over the vocabulary
    col = gW.double().sum(dim=0).abs().max().item()
    scale = gW.double().abs().sum(dim=0).max().item()
    say(f"  max |sum_v grad_W| = {col:.3e} (scale {scale:.3e})")
    assert col <= 1e-3 * scale
    masked = torch.from_numpy(inp.y == -100).to(DEV)
    assert torch.all(gh[masked] == 0)


def test_qwen3_8b_shape_fwd_bwd_sampled():
    _full_shape_check("qwen3_8b")


def test_qwen3_30b_a3b_shape_fwd_bwd_sampled():
    _full_shape_check("qwen3_30b_a3b", n_rows=12, n_vocab=12)


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
