"""Helpers shared by the GPU tests: moving seeded inputs to the device and
comparing against the fp64 oracle."""
import functools
import math
import sys

import numpy as np
import torch

import synth

DEV = torch.device("cuda:0")

# Tolerances fixed by the target: |dlogp| <= 1e-3 absolute, gradients within
# 2e-2 relative L2 (Frobenius norm over the compared tensor, fp64).
LOGP_TOL = 1e-3
GRAD_RTOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def i32_dev(y: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.int32)).to(DEV)


def f32_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_inputs(inp):
    return bf16_dev(inp.h), bf16_dev(inp.W), i32_dev(inp.y), f32_dev(inp.g)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


@functools.lru_cache(maxsize=2)
def config(name: str):
    say(f"[inputs] generating {name}")
    return synth.config(name)


def f32_minus_log(V: int) -> float:
    return float(np.float32(-math.log(V)))


def target_sweep():
    """Targets at every lane / element position of a 256-column tile and at
    the edges: H=128, V=20000, so a split is 625 columns = four full chunks
    and a 113-column chunk, and its third tile holds 113 columns (the second
    128-column wave of that tile has none); both sides of every split edge
    (and so of every aligned block of splits a vocabulary shard can be)."""
    H, V = 128, 20000
    S = -(-V // 32)
    cols = list(range(256))                          # split 0, tile 0: every position
    cols += [256, 383, 384, 511, 512, 600, S - 1]    # tile 1, the short chunk, the split's end
    cols += [31 * S + 511, 31 * S + 512, V - 2, V - 1]
    cols += [c for b in range(1, 32) for c in (b * S - 1, b * S)]  # both sides of every split edge
    y = np.array(cols + [-100, -100], dtype=np.int32)
    inp = synth.make_inputs(len(y), H, V, 0.0, name="target_sweep")
    inp.y = y
    return inp
