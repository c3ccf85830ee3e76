"""Plant plausible mistakes in the oracle and check that the pins catch them.

Each mutant is the oracle's source with one small edit (a dropped term, a
flipped sign, a wrong index or base, an off-by-one range test), loaded as a
separate module.  The pins of tests/test_oracle_pins.py are then run against
it; at least one must fail.  Nothing here touches the real oracle module.
"""
import inspect
import types

import pytest

import oracle.linear_logp as real
import tests.test_oracle_pins as pins

SRC = inspect.getsource(real)

MUTANTS = {
    "decode_shift": ("<< np.uint32(16)).view(np.float32)", "<< np.uint32(15)).view(np.float32)"),
    "lse_drops_max": ("lse_a = m + np.log(s)\n    # target", "lse_a = np.log(s)\n    # target"),
    "log_base_2": ("lse_a = m + np.log(s)\n    # target", "lse_a = m + np.log2(s)\n    # target"),
    "merge_log_base_2": ("lse_a = m + np.log(s)\n    z_t = (ZT", "lse_a = m + np.log2(s)\n    z_t = (ZT"),
    "rescale_sign": ("s = s * np.exp(m - m_new)", "s = s * np.exp(m_new - m)"),
    "target_row_off_by_one": ('z_t = np.einsum("tk,tk->t", Ha, Wm[ya])',
                              'z_t = np.einsum("tk,tk->t", Ha, Wm[(ya + 1) % Wm.shape[0]])'),
    "merge_rescale_sign": ("np.exp(M[:, act] - m)", "np.exp(m - M[:, act])"),
    "ownership_off_by_one": ("(local < n)", "(local <= n)"),
    "dz_sign": ("dZ = -ga[:, None] * P\n        hit", "dZ = ga[:, None] * P\n        hit"),
    "dz_target_sign": ("dZ[rows[hit], ya[hit] - v0] += ga[hit]", "dZ[rows[hit], ya[hit] - v0] -= ga[hit]"),
    "bwd_drops_lse": ("P = np.exp(Ha @ Wb.T - lse[:, None])", "P = np.exp(Ha @ Wb.T)"),
    "grad_W_uses_wrong_operand": ("grad_W[v0:v1] = dZ.T @ Ha", "grad_W[v0:v1] = dZ.T @ (Ha * 0.5)"),
    "grad_h_transposed_block": ("gh_a += dZ @ Wb", "gh_a += (dZ @ Wb)[::-1]"),
}

PIN_TESTS = [
    (pins.test_bf16_decode_known_values, {}),
    (pins.test_p1_zero_input_gives_minus_log_V, {"V": 4096, "which": "h"}),
    (pins.test_p2_one_hot_closed_form, {"V": 4096}),
    (pins.test_p4_matches_library_log_softmax, {}),
    (pins.test_p5_merge_of_ranges_equals_unsharded, {"cuts": [1000, 3500]}),
    (pins.test_p6_finite_differences, {}),
    (pins.test_p6_grad_W_columns_sum_to_zero, {}),
    (pins.test_p6_zero_weight_closed_form, {}),
    (pins.test_p7_masked_rows, {}),
]


def make_mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation site for {name} not unique"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


def test_real_oracle_passes_selected_pins():
    for fn, kw in PIN_TESTS:
        fn(orc=real, **kw)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mut = make_mutant(name)
    caught = []
    for fn, kw in PIN_TESTS:
        try:
            fn(orc=mut, **kw)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(fn.__name__)
    assert caught, f"mutant {name} passed every pin"
