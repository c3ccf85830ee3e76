"""Bit-level record of the numerical contract: sha256 digests of the GPU's
outputs on fixed seeded inputs, one record per contract version.

This is the GPU's own bits, a self-pin (equal contract version and equal
inputs must give equal bits, on every run and every MI355X), never a parity
reference: parity against the fp64 oracle is tested elsewhere.  A kernel
change that alters any bit must come with a new contract version and a new
record (written by record_hashes.py on a GPU).
"""
import hashlib
import json
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
RECORD = os.path.join(HERE, "hashes.json")


def digest(t: torch.Tensor) -> str:
    return hashlib.sha256(t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()).hexdigest()


def compute():
    """{case: {output: sha256}} for every recorded case (needs the GPU)."""
    import selected_token_lm_amd as rlk
    import synth
    from tests.gpu_util import bf16_dev, dev_inputs, f32_dev, i32_dev

    out = {}
    # Qwen3-8B-shaped forward (T=4096, H=4096, V=151936, 15 % of rows ignored)
    inp = synth.config("qwen3_8b")
    h, W, y, _ = dev_inputs(inp)
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    out["qwen3_8b_fwd"] = {"logp": digest(logp), "lse": digest(lse)}
    del h, W, y, logp, lse
    # a small forward + backward (ragged rows and splits, several groups of
    # splits would give the same bits)
    inp = synth.make_inputs(700, 256, 30000, 0.15)
    h, W, y, g = dev_inputs(inp)
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    gh, gW = rlk.linear_logp_bwd(h, W, y, lse, g)
    out["small_fwd_bwd"] = {"logp": digest(logp), "lse": digest(lse), "grad_h": digest(gh),
                            "grad_W": digest(gW)}
    # two vocabulary shards' partial records (S = 938, shard = 16 splits)
    S = -(-inp.V // 32)
    parts = [rlk.lse_partial(h, W[a:a + 16 * S], y, a, inp.V) for a in (0, 16 * S)]
    out["small_partials"] = {"shard0": digest(parts[0]), "shard1": digest(parts[1])}
    # merges of counts that are not powers of two (aligned blocks of 16, 8, 8
    # and of 8, 8, 8, 4, 4 splits)
    for name, widths in (("merge3", (16, 8, 8)), ("merge5", (8, 8, 8, 4, 4))):
        starts = np.cumsum((0,) + widths[:-1])
        ps = [rlk.lse_partial(h, W[a * S:min((a + n) * S, inp.V)], y, int(a * S), inp.V)
              for a, n in zip(starts, widths)]
        lp, ls = rlk.lse_merge(torch.stack(ps), y)
        out["small_partials"][name + "_logp"] = digest(lp)
        out["small_partials"][name + "_lse"] = digest(ls)
    # the RL objective on those log-probabilities
    gen = np.random.Generator(np.random.PCG64(11))
    old = f32_dev(inp_logp_shift(gen, logp.cpu().numpy()))
    adv = f32_dev(gen.standard_normal(inp.T).astype(np.float32))
    ref = f32_dev(inp_logp_shift(gen, logp.cpu().numpy()))
    loss, gl = rlk.rl_token_loss(logp, old, adv, y, 0.2, 0.28, 0.05, ref, 1.0 / 700)
    out["small_rl_loss"] = {"loss": digest(loss), "g": digest(gl)}
    # the dense product (ragged M and N, bf16 and fp32 out)
    A = bf16_dev(synth.normal_bf16(1, 300, 512))
    B = bf16_dev(synth.normal_bf16(2, 700, 512, 1 / 16))
    out["gemm"] = {"f32": digest(rlk.gemm_bf16_nt(A, B)),
                   "bf16": digest(rlk.gemm_bf16_nt(A, B, out_dtype=torch.bfloat16))}
    torch.cuda.synchronize()
    return out


def inp_logp_shift(gen, logp):
    """A nearby 'old policy' log-probability: logp plus N(0, 0.1) noise."""
    return (logp + 0.1 * gen.standard_normal(logp.shape[0])).astype(np.float32)


def load():
    if not os.path.exists(RECORD):
        return {}
    with open(RECORD) as f:
        return json.load(f)
