"""Forward, range partial and merge on the GPU, through the C ABI.

Parity: element by element against the fp64 oracle on the same seeded
inputs (|dlogp| <= 1e-3).  Self-pins that need no oracle: bit-identical
repeats, batch composition / row order invariance, shard merge == unsharded,
and closed forms evaluated on the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import selected_token_lm_amd as rlk
import synth
from tests.gpu_util import (DEV, LOGP_TOL, bf16_dev, config, dev_inputs, f32_minus_log, i32_dev,
                            say, target_sweep, to64)

pytestmark = pytest.mark.gpu


# With every logit 0 the chunk sums are exact integers and s == V exactly, so
# logp = -(log2(V) * ln 2) with the hardware log2 (at most 1 ulp off) and a
# rounded product: 1 ulp of log2 V (scaled by ln 2 < 1) + the error of the
# fp32 ln 2 (3e-8 here) + half an ulp of rounding stays below 2 ulp of ln V.
P1_ULPS = 2


def run_fwd(inp):
    h, W, y, _ = dev_inputs(inp)
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    torch.cuda.synchronize()
    return logp, lse


def check_vs_oracle(inp, logp, lse, rows=None):
    rows = np.arange(inp.T) if rows is None else np.asarray(rows)
    ref_logp, ref_lse = oracle.forward(inp.h[rows], inp.W, inp.y[rows])
    got = to64(logp)[rows]
    got_lse = to64(lse)[rows]
    err = np.max(np.abs(got - ref_logp)) if len(rows) else 0.0
    err_lse = np.max(np.abs(got_lse - ref_lse)) if len(rows) else 0.0
    say(f"  max|dlogp|={err:.3e} max|dlse|={err_lse:.3e} over {len(rows)} rows")
    assert err <= LOGP_TOL
    assert err_lse <= LOGP_TOL
    masked = inp.y[rows] == -100
    assert np.all(got[masked] == 0.0) and np.all(got_lse[masked] == 0.0)
    return err


def test_tiny_config_matches_oracle():
    inp = config("tiny")
    say("tiny 64x256x4096")
    logp, lse = run_fwd(inp)
    check_vs_oracle(inp, logp, lse)


@pytest.mark.parametrize("T,H,V,mask", [
    (300, 192, 20000, 0.15),   # ragged rows and a short last chunk per split
    (1, 64, 5003, 0.0),        # one row; V not a multiple of 32
    (129, 128, 257, 0.3),      # splits of 9 columns, one chunk each
    (64, 64, 100, 0.0),        # V < 128: splits of 4 columns, the last 7 splits empty
    (1000, 320, 33000, 0.15),  # 1032-column splits: 8 full chunks + an 8-column chunk
])
def test_ragged_shapes_match_oracle(T, H, V, mask):
    say(f"ragged T={T} H={H} V={V}")
    inp = synth.make_inputs(T, H, V, mask)
    logp, lse = run_fwd(inp)
    check_vs_oracle(inp, logp, lse)


@pytest.mark.parametrize("rows", [None, 64])
def test_target_at_every_tile_position(rows):
    inp = target_sweep()
    if rows is not None:  # a small batch takes the kernel instance for at most 96 rows
        inp.h, inp.y, inp.g, inp.T = inp.h[:rows], inp.y[:rows], inp.g[:rows], rows
    say(f"target sweep T={inp.T} H={inp.H} V={inp.V}")
    logp, lse = run_fwd(inp)
    check_vs_oracle(inp, logp, lse)


def test_all_rows_masked_and_empty_batch():
    inp = synth.make_inputs(70, 64, 1000, 0.0)
    inp.y[:] = -100
    logp, lse = run_fwd(inp)
    assert torch.all(logp == 0) and torch.all(lse == 0)
    h = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    W = bf16_dev(inp.W)
    y = torch.empty(0, dtype=torch.int32, device=DEV)
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    assert logp.numel() == 0


def test_zero_hidden_closed_form():
    # every logit is exactly 0: chunk sums are exact integers, s == V exactly
    for V in (4096, 151936):
        T, H = 130, 128
        h = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
        W = bf16_dev(synth.normal_bf16(2, V, H, 0.1))
        y = i32_dev(synth.targets(T, V, 0.1))
        logp, lse = rlk.linear_logp_fwd(h, W, y)
        part = rlk.lse_partial(h, W, y, 0, V)
        torch.cuda.synchronize()
        act = (y != -100)
        want = f32_minus_log(V)
        got = logp[act].double()
        say(f"  V={V}: logp range [{got.min().item():.9f}, {got.max().item():.9f}] want {want:.9f}")
        ulps = ((got - want).abs() / float(np.spacing(np.float32(abs(want))))).max().item()
        say(f"  V={V}: {ulps:.2f} ulp from the fp32 -ln V")
        assert ulps <= P1_ULPS
        assert torch.all(part[act, 0] == 0.0) and torch.all(part[act, 1] == float(V))


@pytest.mark.parametrize("V", [4096, 151936])
def test_one_hot_closed_form(V):
    H = 64
    v0 = 3 if V == 4096 else 100_000
    for alpha, bits in ((1.0, 0x3F80), (8.0, 0x4100), (40.0, 0x4220)):
        h = np.zeros((2, H), np.uint16)
        h[:, 0] = 0x3F80
        Wn = np.zeros((V, H), np.uint16)
        Wn[v0, 0] = bits
        y = np.array([v0, (v0 + 7) % V], np.int32)
        logp, _ = rlk.linear_logp_fwd(bf16_dev(h), bf16_dev(Wn), i32_dev(y))
        got = to64(logp)
        c = math.log1p((V - 1) * math.exp(-alpha))
        say(f"  V={V} alpha={alpha}: {got} vs {[-c, -alpha - c]}")
        assert abs(got[0] + c) <= 1e-5
        assert abs(got[1] + alpha + c) <= 1e-5


def test_identical_rows_and_columns_give_identical_bits():
    # MFMA position invariance: one hidden row at every row position of two
    # tiles, and one weight row at every column position of every chunk.
    H, V = 256, 20000
    hrow = synth.normal_bf16(1, 1, H)
    h = bf16_dev(np.repeat(hrow, 256, axis=0))
    W = bf16_dev(synth.normal_bf16(2, V, H, 1 / 16))
    y = i32_dev(synth.targets(256, V, 0.0))
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    assert torch.all(lse == lse[0])
    Wrow = synth.normal_bf16(2, 1, H, 1 / 16)
    W1 = bf16_dev(np.repeat(Wrow, V, axis=0))
    h2 = bf16_dev(synth.normal_bf16(1, 256, H))
    logp, lse = rlk.linear_logp_fwd(h2, W1, y)
    torch.cuda.synchronize()
    # all logits of a row equal: every exp is exactly 1, s == V, logp == -ln V
    want = f32_minus_log(V)
    assert torch.all((logp.double() - want).abs() <= P1_ULPS * np.spacing(np.float32(abs(want))))


def test_out_of_range_target_gives_nan():
    inp = synth.make_inputs(10, 64, 500, 0.0)
    inp.y[3] = 500
    inp.y[5] = -7
    logp, lse = run_fwd(inp)
    got = logp.cpu().numpy()
    assert np.isnan(got[3]) and np.isnan(got[5])
    assert np.all(np.isfinite(np.delete(got, [3, 5])))


def test_bitwise_repeat():
    inp = synth.make_inputs(500, 256, 30000, 0.15)
    h, W, y, _ = dev_inputs(inp)
    a, la = rlk.linear_logp_fwd(h, W, y)
    for _ in range(9):
        b, lb = rlk.linear_logp_fwd(h, W, y)
        assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("sweep", [False, True])
def test_partial_and_merge_match_forward_bitwise(sweep):
    # V = 20000, S = 625; the sweep puts targets at every tile position and on
    # the edges of splits and of the shards (the first and last row of each)
    inp = target_sweep() if sweep else synth.make_inputs(300, 128, 20000, 0.15)
    h, W, y, _ = dev_inputs(inp)
    ref, ref_lse = rlk.linear_logp_fwd(h, W, y)
    V, S = inp.V, 625
    for P in (1, 2, 4, 8, 32):
        width = 32 // P * S
        parts = [rlk.lse_partial(h, W[a:min(a + width, V)], y, a, V) for a in range(0, V, width)]
        assert len(parts) == P
        logp, lse = rlk.lse_merge(torch.stack(parts), y)
        assert torch.equal(logp, ref), P
        assert torch.equal(lse, ref_lse), P
    # the partial statistics themselves agree with the oracle's range statistics
    parts = [rlk.lse_partial(h, W[a:a + 32 // 2 * S], y, a, V) for a in (0, 16 * S)]
    for a, p in zip((0, 16 * S), parts):
        ref_p = oracle.partial(inp.h, inp.W[a:a + 16 * S], inp.y, a)
        got = p.cpu().numpy().astype(np.float64)
        owned = p.cpu().view(torch.int32)[:, 3].numpy().astype(bool)
        act = inp.y != -100
        assert np.array_equal(owned, ref_p["owned"])
        # s is relative to m: compare m and log(s) + m
        assert np.max(np.abs(got[act, 0] - ref_p["m"][act])) <= 1e-4
        lse_got = got[act, 0] + np.log(got[act, 1])
        lse_ref = ref_p["m"][act] + np.log(ref_p["s"][act])
        assert np.max(np.abs(lse_got - lse_ref)) <= 1e-3
        assert np.max(np.abs(got[owned, 2] - ref_p["z_t"][owned])) <= 1e-4


def test_merge_rejects_ownerless_rows():
    inp = synth.make_inputs(50, 64, 1000, 0.0)
    h, W, y, _ = dev_inputs(inp)
    p0 = rlk.lse_partial(h, W[:512], y, 0, 1000)  # S = 32: 16 splits = 512 rows
    logp, _ = rlk.lse_merge(p0[None], y)  # the upper half is missing
    owned = inp.y < 512
    got = logp.cpu().numpy()
    assert np.all(np.isnan(got[~owned])) and np.all(np.isfinite(got[owned]))


def test_batch_composition_invariance_small():
    inp = synth.make_inputs(700, 128, 12000, 0.15)
    h, W, y, _ = dev_inputs(inp)
    ref, ref_lse = rlk.linear_logp_fwd(h, W, y)
    plan = synth.rebatch_plan(700, sizes=(1, 7, 128, 300, 900))
    for rows in plan:
        r = torch.from_numpy(rows).to(DEV)
        logp, lse = rlk.linear_logp_fwd(h[r], W, y[r])
        assert torch.equal(logp, ref[r]) and torch.equal(lse, ref_lse[r]), len(rows)


@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 128, 129])
def test_small_batches_bitwise_equal_to_large_batch(n):
    # batches of at most 96 rows run with the idle row blocks switched off;
    # every row must still get the bits of the same row in a large batch
    inp = synth.make_inputs(400, 576, 9000, 0.15)
    h, W, y, _ = dev_inputs(inp)
    ref, ref_lse = rlk.linear_logp_fwd(h, W, y)
    rows = np.random.Generator(np.random.PCG64(n)).permutation(inp.T)[:n]
    r = torch.from_numpy(rows).to(DEV)
    say(f"[fwd] small batch of {n} rows ({int((inp.y[rows] != -100).sum())} active)")
    logp, lse = rlk.linear_logp_fwd(h[r].contiguous(), W, y[r].contiguous())
    assert torch.equal(logp, ref[r]) and torch.equal(lse, ref_lse[r])
    check_vs_oracle(inp, ref, ref_lse, rows[:8])


# --- full-size Qwen3-8B-shaped LM head (T=4096, H=4096, V=151936, 15% masked) ---

@pytest.fixture(scope="module")
def q8b():
    inp = config("qwen3_8b")
    h, W, y, _ = dev_inputs(inp)
    logp, lse = rlk.linear_logp_fwd(h, W, y)
    torch.cuda.synchronize()
    return inp, h, W, y, logp, lse


def test_qwen3_8b_two_shard_merge_bitwise(q8b):
    inp, h, W, y, logp, lse = q8b
    half = 75968
    p0 = rlk.lse_partial(h, W[:half], y, 0, inp.V)
    p1 = rlk.lse_partial(h, W[half:], y, half, inp.V)
    m, ml = rlk.lse_merge(torch.stack([p0, p1]), y)
    assert torch.equal(m, logp) and torch.equal(ml, lse)
    one = rlk.lse_partial(h, W, y, 0, inp.V)
    m1, _ = rlk.lse_merge(one[None], y)
    assert torch.equal(m1, logp)


def test_qwen3_8b_rebatch_bitwise(q8b):
    inp, h, W, y, logp, lse = q8b
    plan = synth.rebatch_plan(inp.T)
    for rows in plan:
        r = torch.from_numpy(rows).to(DEV)
        got, gl = rlk.linear_logp_fwd(h[r], W, y[r])
        assert torch.equal(got, logp[r]) and torch.equal(gl, lse[r]), len(rows)


def test_qwen3_8b_heavy_tail_rebatch_bitwise(q8b):
    inp, h, W, y, logp, lse = q8b
    h8 = h * 8  # exact: power-of-two scale of bf16 values
    ref, ref_lse = rlk.linear_logp_fwd(h8, W, y)
    rows = np.random.Generator(np.random.PCG64(8)).choice(inp.T, 24, replace=False)
    h8_bits = synth.scale_bf16(inp.h[rows], 8.0)
    ref_o, _ = oracle.forward(h8_bits, inp.W, inp.y[rows])
    err = np.max(np.abs(to64(ref)[rows] - ref_o))
    say(f"  heavy tail x8: max|dlogp|={err:.3e}, max|lse|={ref_lse.abs().max().item():.1f}")
    assert err <= LOGP_TOL
    for rows in synth.rebatch_plan(inp.T):
        r = torch.from_numpy(rows).to(DEV)
        got, gl = rlk.linear_logp_fwd(h8[r], W, y[r])
        assert torch.equal(got, ref[r]) and torch.equal(gl, ref_lse[r]), len(rows)


@pytest.mark.parametrize("T,H,V", [(3, 65536, 600), (5, 64, 8_000_000)])
def test_maximum_hidden_and_vocabulary(T, H, V):
    # the largest H and V the library accepts (32-bit offsets at their limits)
    say(f"max sizes T={T} H={H} V={V}")
    inp = synth.make_inputs(T, H, V, 0.0)
    logp, lse = run_fwd(inp)
    check_vs_oracle(inp, logp, lse)


def test_brute_force_every_target_sums_to_one():
    """Pin P3 on the GPU: 8 rows of the tiny configuration, each repeated with
    every one of the V = 4096 targets, as one 32768-row batch.  The
    probabilities of a row over all targets sum to 1, and every copy of a row
    has the same lse bits (its batch-mates do not matter)."""
    inp = config("tiny")
    rows = np.arange(8) * 7
    V = inp.V
    h = bf16_dev(np.repeat(inp.h[rows], V, axis=0))
    y = i32_dev(np.tile(np.arange(V, dtype=np.int32), len(rows)))
    logp, lse = rlk.linear_logp_fwd(h, bf16_dev(inp.W), y)
    torch.cuda.synchronize()
    lp = to64(logp).reshape(len(rows), V)
    ls = lse.cpu().view(torch.int32).numpy().reshape(len(rows), V)
    sums = np.exp(lp).sum(axis=1)
    say(f"  sum_v exp(logp_v) - 1 per row: {np.array2string(sums - 1, precision=2)}")
    assert np.all(np.abs(sums - 1.0) <= 1e-4)
    assert np.all(ls == ls[:, :1])
