"""Batches whose row counts exceed what one grid dimension of a launch holds
(at most 2^31 - 1 threads along x, 65535 along y): the row-wise kernels
stride over their rows, and the results still match the oracle."""
import numpy as np
import pytest
import torch

import oracle
import selected_token_lm_amd as rlk
import synth
from tests.gpu_util import DEV, GRAD_RTOL, LOGP_TOL, dev_inputs, rel_l2, say, to64

pytestmark = pytest.mark.gpu


def test_saved_logits_backward_past_65535_rows():
    # dz from saved logits strides over more rows than grid.y holds
    T, H, V = 66000, 64, 300
    say(f"saved logits past 65535 rows: T={T} H={H} V={V}")
    inp = synth.make_inputs(T, H, V, 0.15)
    h, W, y, g = dev_inputs(inp)
    logp, lse, zs = rlk.linear_logp_fwd_save(h, W, y)
    gh_s, gW_s = rlk.linear_logp_bwd_saved(h, W, y, lse, g, zs)
    gh_r, gW_r = rlk.linear_logp_bwd(h, W, y, lse, g)
    torch.cuda.synchronize()
    assert torch.equal(gh_s, gh_r) and torch.equal(gW_s, gW_r)
    ref_gh, ref_gW = oracle.backward(inp.h, inp.W, inp.y, inp.g)
    e_h, e_W = rel_l2(to64(gh_s), ref_gh), rel_l2(to64(gW_s), ref_gW)
    say(f"  relL2 grad_h={e_h:.2e} grad_W={e_W:.2e}")
    assert e_h <= GRAD_RTOL and e_W <= GRAD_RTOL


def test_forward_backward_past_2_22_rows():
    # more rows than the row-wise kernels' 2^22 blocks: gathering the active
    # rows and zeroing the ignored rows' gradients stride over the rest
    T, H, V = (1 << 22) + 300, 64, 64
    say(f"rows past 2^22: T={T} H={H} V={V}")
    inp = synth.make_inputs(T, H, V, 0.15)
    h, W, y, g = dev_inputs(inp)
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    gh, _ = rlk.linear_logp_bwd(h, W, y, lse, g, need_grad_W=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(T, 2000, replace=False), np.arange(T - 300, T)]))
    rows_dev = torch.from_numpy(rows).to(DEV)
    ref_logp, ref_lse = oracle.forward(inp.h[rows], inp.W, inp.y[rows])
    err = float(np.max(np.abs(to64(logp[rows_dev]) - ref_logp)))
    err_lse = float(np.max(np.abs(to64(lse[rows_dev]) - ref_lse)))
    e_h = rel_l2(to64(gh[rows_dev]), oracle.backward_rows(inp.h, inp.W, inp.y, inp.g, rows))
    ignored = torch.from_numpy(inp.y == -100).to(DEV)
    say(f"  {len(rows)} sampled rows: max|dlogp|={err:.2e} max|dlse|={err_lse:.2e} relL2 grad_h={e_h:.2e}")
    assert err <= LOGP_TOL and err_lse <= LOGP_TOL and e_h <= GRAD_RTOL
    assert int(torch.count_nonzero(gh[ignored])) == 0
    assert bool(torch.all(logp[ignored] == 0))
