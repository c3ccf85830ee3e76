"""The operator under HIP graph capture (torch.cuda.graph), through the C ABI.

Every entry point only enqueues kernels on the caller's stream: no
allocation, no memset, no synchronisation.  So a captured forward +
backward must replay to the eager results bit for bit, read its inputs at
replay time (new values copied into the captured buffers give the eager
results of the new values), and keep doing so across replays separated by
unrelated eager work and synchronisations.
"""
import numpy as np
import pytest
import torch

import selected_token_lm_amd as rlk
import synth
from tests.gpu_util import DEV, bf16_dev, dev_inputs, say

pytestmark = pytest.mark.gpu


def eager(h, W, y, g):
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    gh, gW = rlk.linear_logp_bwd(h, W, y, lse, g)
    torch.cuda.synchronize()
    return logp, lse, gh, gW


def test_captured_forward_backward_replays_bitwise():
    T, H, V = 300, 256, 5000
    inp = synth.make_inputs(T, H, V, 0.15)
    h, W, y, g = dev_inputs(inp)
    ref = eager(h, W, y, g)
    ws_f = torch.empty(rlk.workspace_bytes(rlk.OP_FWD, T, H, V), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(rlk.workspace_bytes(rlk.OP_BWD, T, H, V), dtype=torch.uint8, device=DEV)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's kind, as torch asks
        logp, lse = rlk.linear_logp_fwd(h, W, y, ws=ws_f)
        rlk.linear_logp_bwd(h, W, y, lse, g, ws=ws_b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        c_logp, c_lse = rlk.linear_logp_fwd(h, W, y, ws=ws_f)
        c_gh, c_gW = rlk.linear_logp_bwd(h, W, y, c_lse, g, ws=ws_b)
    torch.cuda.synchronize()

    other = synth.make_inputs(T, H, V, 0.3, h_scale=2.0)
    o_h, o_W, o_y, o_g = dev_inputs(other)
    for rep in range(3):
        say(f"[graph] replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((c_logp, c_lse, c_gh, c_gW), ref):
            assert torch.equal(got, want)
        # unrelated eager work (the library's own kernels on other data) in between
        eager(o_h, o_W, o_y, o_g)

    # new values in the captured input buffers: the replay computes on them
    new = synth.make_inputs(T, H, V, 0.3, h_scale=2.0)
    h.copy_(bf16_dev(new.h))
    y.copy_(torch.from_numpy(new.y).to(DEV))
    torch.cuda.synchronize()
    want = eager(h, W, y, g)
    for rep in range(2):
        graph.replay()
        torch.cuda.synchronize()
        for got, w in zip((c_logp, c_lse, c_gh, c_gW), want):
            assert torch.equal(got, w)
    assert not torch.equal(want[0], ref[0])
