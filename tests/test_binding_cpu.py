"""The Python binding rejects malformed per-row tensors before any kernel
runs (CPU only: every call below fails on its shapes, before the device
check, so no GPU is needed).

The kernels read element t of y, lse, g, logp_old, adv and logp_ref for
every row t < T; a shorter tensor would be read past its end on the device,
so the binding checks every per-row length against T.
"""
import pytest
import torch

import selected_token_lm_amd as rlk

T, H, V = 8, 64, 100


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(n):
    return torch.zeros(n, dtype=torch.float32)


def i32(n):
    return torch.zeros(n, dtype=torch.int32)


def test_forward_target_length_and_dtype():
    with pytest.raises(ValueError, match="y must be"):
        rlk.linear_logp_fwd(bf(T, H), bf(V, H), i32(T - 1))
    with pytest.raises(ValueError, match="y must be"):
        rlk.linear_logp_fwd(bf(T, H), bf(V, H), i32(T).reshape(2, 4))
    with pytest.raises(TypeError, match="int32 or int64"):
        rlk.linear_logp_fwd(bf(T, H), bf(V, H), torch.zeros(T, dtype=torch.float32))
    with pytest.raises(TypeError, match="bfloat16"):
        rlk.linear_logp_fwd(torch.zeros(T, H), bf(V, H), i32(T))
    with pytest.raises(ValueError, match=r"\[T, H\]"):
        rlk.linear_logp_fwd(bf(T, H), bf(V, H + 64), i32(T))
    # well-formed CPU tensors get as far as the device check
    with pytest.raises(ValueError, match="device tensors"):
        rlk.linear_logp_fwd(bf(T, H), bf(V, H), i32(T))


@pytest.mark.parametrize("which", ["lse", "g"])
@pytest.mark.parametrize("n", [T - 1, T + 1])
def test_backward_rejects_short_or_long_row_tensors(monkeypatch, which, n):
    # get past the device check of h, W, y with a stand-in that only reports
    # CPU tensors as device tensors; the per-row check must still fire first
    monkeypatch.setattr(rlk, "_prep", lambda h, W, y: (h, W, y))
    args = {"lse": f32(T), "g": f32(T)}
    args[which] = f32(n)
    for fn in (lambda: rlk.linear_logp_bwd(bf(T, H), bf(V, H), i32(T), args["lse"], args["g"]),
               lambda: rlk.linear_logp_bwd_saved(bf(T, H), bf(V, H), i32(T), args["lse"], args["g"],
                                                 torch.zeros((T, 4), dtype=torch.float32))):
        with pytest.raises(ValueError, match=f"{which} must be 1-D of length T = {T}"):
            fn()


def test_merge_rejects_target_length():
    parts = torch.zeros((2, T, 4), dtype=torch.float32)
    with pytest.raises(ValueError, match="device tensor"):
        rlk.lse_merge(parts, i32(T))
    with pytest.raises(ValueError, match="parts must be"):
        rlk.lse_merge(torch.zeros((2, T, 3), dtype=torch.float32), i32(T))


@pytest.mark.parametrize("bad", ["logp_old", "adv", "y", "logp_ref"])
def test_rl_loss_rejects_mismatched_lengths(bad):
    kw = dict(logp_old=f32(T), adv=f32(T), y=i32(T), logp_ref=f32(T))
    kw[bad] = (i32 if bad == "y" else f32)(T - 2)
    with pytest.raises(ValueError, match=f"{bad} must be 1-D of length T = {T}"):
        rlk.rl_token_loss(f32(T), kw["logp_old"], kw["adv"], kw["y"], beta=0.1, logp_ref=kw["logp_ref"])
    with pytest.raises(ValueError, match="logp_ref is required"):
        rlk.rl_token_loss(f32(T), f32(T), f32(T), i32(T), beta=0.1)
