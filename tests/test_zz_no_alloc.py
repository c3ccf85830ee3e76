"""The forward entry point that allocates nothing (rlk_linear_logp_fwd_noalloc):
its workspace is the library's fixed device scratch.  Output must equal the
workspace entry point's bit for bit (the same kernels); two calls in a row,
the second smaller, check that nothing of the first call's scratch contents
leaks into the second; sizes beyond the scratch are refused on the host."""
import numpy as np
import pytest
import torch

import selected_token_lm_amd as rlk
import synth
from tests.gpu_util import DEV, dev_inputs, say

pytestmark = pytest.mark.gpu


def _both(inp):
    h, W, y, _ = dev_inputs(inp)
    ref, ref_lse = rlk.linear_logp_fwd(h, W, y)
    got, got_lse = rlk.linear_logp_fwd_noalloc(h, W, y)
    torch.cuda.synchronize()
    return ref, ref_lse, got, got_lse


def test_noalloc_equals_workspace_entry_point_twice():
    big = synth.make_inputs(1500, 512, 40000, 0.15)
    small = synth.make_inputs(300, 256, 20000, 0.3)
    for inp in (big, small):
        say(f"[noalloc] T={inp.T} H={inp.H} V={inp.V}: "
            f"{rlk.workspace_bytes(rlk.OP_FWD, inp.T, inp.H, inp.V)} of {rlk.NOALLOC_SCRATCH_BYTES} scratch bytes")
        ref, ref_lse, got, got_lse = _both(inp)
        assert torch.equal(got, ref) and torch.equal(got_lse, ref_lse)
        assert np.all(np.isfinite(got.cpu().numpy()))


def test_noalloc_refuses_sizes_beyond_the_scratch():
    T, H, V = 4096, 4096, 151936   # ~74 MB of workspace
    assert rlk.workspace_bytes(rlk.OP_FWD, T, H, V) > rlk.NOALLOC_SCRATCH_BYTES
    h = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((V, H), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros(T, dtype=torch.int32, device=DEV)
    with pytest.raises(rlk.RlkError, match="fixed device scratch"):
        rlk.linear_logp_fwd_noalloc(h, W, y)
