"""The seeded input generator: determinism, rounding and the workload recipe."""
import numpy as np

import synth


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, -one - 3 * ulp / 4,
                  np.float32(40.0), np.float32(3.0e-39)], np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    # ties go to the even mantissa: 1+ulp/2 -> 1, 1+3ulp/2 -> 1+2ulp
    want = np.array([1.0, 1.0, 1.0 + 2 * ulp, 1.0, -(1.0 + ulp), 40.0, np.nan], np.float32)
    assert np.array_equal(got[:6], want[:6])
    # a denormal survives as the nearest bf16 denormal
    assert got[6] > 0 and abs(got[6] - 3.0e-39) < 2.0 ** -133


def test_generator_is_deterministic_and_blockwise():
    a = synth.normal_bf16(2, 3000, 64, 0.125)
    b = synth.normal_bf16(2, 3000, 64, 0.125)
    assert np.array_equal(a, b)
    # the first block does not depend on how many rows follow it
    c = synth.normal_bf16(2, 100, 64, 0.125)
    assert np.array_equal(a[:100], c)
    assert not np.array_equal(a, synth.normal_bf16(3, 3000, 64, 0.125))


def test_moments_match_recipe():
    inp = synth.make_inputs(2048, 256, 2000, 0.15)
    h = synth.bf16_bits_to_f32(inp.h).astype(np.float64)
    W = synth.bf16_bits_to_f32(inp.W).astype(np.float64)
    assert abs(h.mean()) < 0.01 and abs(h.std() - 1.0) < 0.01
    assert abs(W.std() * np.sqrt(inp.H) - 1.0) < 0.01
    z = h[:64] @ W.T
    assert abs(z.std() - 1.0) < 0.05


def test_mask_count_and_target_range():
    y = synth.targets(4096, 151936, 0.15)
    assert (y == -100).sum() == 614
    act = y[y != -100]
    assert act.min() >= 0 and act.max() < 151936
    y2 = synth.targets(16384, 151936, 0.15)
    assert (y2 == -100).sum() == 2458
    assert (synth.targets(64, 4096, 0.0) == -100).sum() == 0


def test_power_of_two_scale_is_exact():
    h = synth.normal_bf16(1, 50, 32)
    h8 = synth.scale_bf16(h, 8.0)
    assert np.array_equal(synth.bf16_bits_to_f32(h8), synth.bf16_bits_to_f32(h) * 8)


def test_rebatch_plan():
    plan = synth.rebatch_plan(4096)
    assert sorted(len(b) for b in plan) == [1, 7, 128, 1000, 8192]
    allrows = np.concatenate(plan)
    assert allrows.min() >= 0 and allrows.max() < 4096
    # the 9328 rows are a prefix of a stream of full permutations
    assert len(np.unique(allrows)) == 4096
    assert [len(b) for b in plan] == [len(b) for b in synth.rebatch_plan(4096)]
