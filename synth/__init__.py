"""Seeded synthetic inputs for the selected-token log-probability operator.

This module only draws random numbers and lays them out; it holds none of
the operator's arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP
path (``selected_token_lm_amd``) consume what it produces, so the two sides
always see the same input bits.

Recipe (the shapes and distributions of the workloads described on the
RL-Kernel pages: Qwen3-8B-like and Qwen3-30B-A3B-like LM heads):

* ``h``  [T, H] bf16, entries N(0, 1).
* ``W``  [V, H] bf16, entries N(0, std = 1/sqrt(H)), so logits are ~N(0, 1).
* ``y``  [T] int32, uniform in [0, V); a fixed fraction of rows (the first
  ones of a seeded permutation) is set to the ignore value -100.
* ``g``  [T] fp32, N(0, 1): the upstream gradient dL/dlogp.

Random draws happen in fp32 and are rounded to bf16 with round-to-nearest-
even.  Large matrices are drawn in row blocks of ``ROW_BLOCK`` rows, block
``i`` from ``SeedSequence(seed, spawn_key=(i,))``, so the bits do not depend
on the number of threads and any block can be regenerated alone.

Seeds: h=1, W=2, targets=3, mask=4, g=5, re-batching permutations=6.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

IGNORE_INDEX = -100
ROW_BLOCK = 1024

SEED_H, SEED_W, SEED_Y, SEED_MASK, SEED_G, SEED_PERM = 1, 2, 3, 4, 5, 6


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the uint16 bits.

    Inputs here are finite normal draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, rows: int, cols: int, std: float = 1.0) -> np.ndarray:
    """[rows, cols] bf16 bits of N(0, std) draws, drawn in seeded row blocks."""
    out = np.empty((rows, cols), dtype=np.uint16)
    if rows == 0 or cols == 0:
        return out
    nblk = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    scale = np.float32(std)

    def work(i: int) -> None:
        r0 = i * ROW_BLOCK
        r1 = min(rows, r0 + ROW_BLOCK)
        gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(i,))))
        x = gen.standard_normal(size=(r1 - r0, cols), dtype=np.float32)
        if scale != np.float32(1.0):
            x *= scale
        out[r0:r1] = f32_to_bf16_bits(x)

    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))
    return out


def targets(T: int, V: int, mask_frac: float, seed_y: int = SEED_Y, seed_mask: int = SEED_MASK) -> np.ndarray:
    """[T] int32 targets uniform in [0, V); round(mask_frac*T) rows set to -100."""
    y = np.random.Generator(np.random.PCG64(seed_y)).integers(0, V, size=T, dtype=np.int64).astype(np.int32)
    n_mask = int(round(mask_frac * T))
    if n_mask:
        perm = np.random.Generator(np.random.PCG64(seed_mask)).permutation(T)
        y[perm[:n_mask]] = IGNORE_INDEX
    return y


def upstream_grad(T: int, seed: int = SEED_G) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(size=T, dtype=np.float32)


@dataclass
class Inputs:
    name: str
    T: int
    H: int
    V: int
    h: np.ndarray  # uint16 [T, H] bf16 bits
    W: np.ndarray  # uint16 [V, H] bf16 bits
    y: np.ndarray  # int32 [T]
    g: np.ndarray  # float32 [T]
    mask_frac: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def n_active(self) -> int:
        return int(np.count_nonzero(self.y != IGNORE_INDEX))


def make_inputs(T: int, H: int, V: int, mask_frac: float = 0.0, name: str = "custom",
                w_std: float | None = None, h_scale: float = 1.0) -> Inputs:
    """Inputs of the standard recipe at an arbitrary shape."""
    std = np.float32(1.0 / np.sqrt(H)) if w_std is None else np.float32(w_std)
    h = normal_bf16(SEED_H, T, H, 1.0)
    if h_scale != 1.0:
        h = scale_bf16(h, h_scale)
    W = normal_bf16(SEED_W, V, H, float(std))
    y = targets(T, V, mask_frac)
    g = upstream_grad(T)
    return Inputs(name, T, H, V, h, W, y, g, mask_frac)


def scale_bf16(bits: np.ndarray, factor: float) -> np.ndarray:
    """Multiply bf16 values by a power of two (exact for the normal range)."""
    f = np.float32(factor)
    m, e = np.frexp(f)
    if m != 0.5:
        raise ValueError("only power-of-two scales are exact")
    return f32_to_bf16_bits(bf16_bits_to_f32(bits) * f)


# Named workloads.  Shapes: (T, H, V, masked fraction).
CONFIGS = {
    # small parity case: the oracle finishes in well under a second
    "tiny": (64, 256, 4096, 0.0),
    # Qwen3-8B-shaped LM head, forward
    "qwen3_8b": (4096, 4096, 151936, 0.15),
    # Qwen3-30B-A3B-shaped LM head, forward + backward
    "qwen3_30b_a3b": (16384, 2048, 151936, 0.15),
}


def config(name: str) -> Inputs:
    T, H, V, mf = CONFIGS[name]
    return make_inputs(T, H, V, mf, name=name)


REBATCH_SIZES = (1, 7, 128, 1000, 8192)


def rebatch_plan(T: int, sizes=REBATCH_SIZES, seed: int = SEED_PERM):
    """Ragged re-batching of row indices of a T-row batch.

    Rows come from a stream of seeded permutations of range(T), concatenated
    until sum(sizes) rows are drawn (so batches larger than T hold rows more
    than once).  The batches are then emitted in a seeded shuffled order.
    Returns a list of int64 index arrays.
    """
    gen = np.random.Generator(np.random.PCG64(seed))
    need = int(sum(sizes))
    stream = []
    while sum(len(s) for s in stream) < need:
        stream.append(gen.permutation(T))
    rows = np.concatenate(stream)[:need]
    batches = []
    pos = 0
    for s in sizes:
        batches.append(rows[pos:pos + s].astype(np.int64))
        pos += s
    order = gen.permutation(len(batches))
    return [batches[i] for i in order]
