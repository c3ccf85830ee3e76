"""Pins of the fp64 oracle against facts fixed by the mathematics.

The pages print no worked example for this operator, so every pin here is a
closed form, a brute-force identity, a library routine or a finite
difference.  Each is chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a wrong log base) breaks
at least one of them; tests/test_oracle_mutants.py plants such slips and
checks that they are caught.
"""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle as _oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.txt")

BF16_ONE = 0x3F80


@pytest.fixture
def orc():
    """The oracle module under test (tests/test_oracle_mutants.py passes mutants)."""
    return _oracle


def bf16(x):
    """bf16 bits of values exactly representable in bf16."""
    b = synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(b), np.asarray(x, dtype=np.float32))
    return b


def load_golden():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            kind, V, alpha, which, val = line.split()
            out.append((kind, int(V), float(alpha), which, float(val)))
    return out


def test_golden_file_matches_formulas():
    for kind, V, alpha, which, val in load_golden():
        if kind == "uniform":
            assert val == -math.log(V)
        else:
            c = math.log1p((V - 1) * math.exp(-alpha))
            assert val == (-c if which == "target" else -alpha - c)


def test_bf16_decode_known_values(orc):
    bits = np.array([0x3F80, 0xC000, 0x4220, 0x0000, 0x8000, 0x0001, 0x7F7F, 0x3F81], np.uint16)
    want = [1.0, -2.0, 40.0, 0.0, -0.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 1 + 2 ** -7]
    got = orc.bf16_to_f64(bits)
    assert got.dtype == np.float64
    assert list(got) == want


# -- P1: all logits equal ------------------------------------------------------

@pytest.mark.parametrize("V", [4096, 151936])
@pytest.mark.parametrize("which", ["h", "W"])
def test_p1_zero_input_gives_minus_log_V(V, which, orc):
    T, H = 5, 32
    h = np.zeros((T, H), np.uint16) if which == "h" else synth.normal_bf16(1, T, H)
    W = np.zeros((V, H), np.uint16) if which == "W" else synth.normal_bf16(2, V, H, 0.2)
    y = np.array([0, 1, V - 1, 17, V // 2], np.int32)
    logp, lse = orc.forward(h, W, y)
    gold = {(k, v): val for k, v, a, w, val in load_golden() if k == "uniform"}
    expect = gold[("uniform", V)]
    assert np.all(np.abs(logp - expect) <= 1e-13)
    assert np.all(np.abs(lse - math.log(V)) <= 1e-13)


# -- P2: one-hot logits, heavy tail ---------------------------------------------

@pytest.mark.parametrize("V", [4096, 151936])
def test_p2_one_hot_closed_form(V, orc):
    H = 32
    v0 = 3 if V == 4096 else 100_000
    rows = [r for r in load_golden() if r[0] == "onehot" and r[1] == V]
    for alpha in (1.0, 8.0, 40.0):
        h = np.zeros((2, H), np.uint16)
        h[:, 0] = BF16_ONE
        W = np.zeros((V, H), np.uint16)
        W[v0, 0] = bf16([alpha])[0]
        y = np.array([v0, (v0 + 7) % V], np.int32)
        logp, lse = orc.forward(h, W, y)
        exp_t = [r[4] for r in rows if r[2] == alpha and r[3] == "target"][0]
        exp_o = [r[4] for r in rows if r[2] == alpha and r[3] == "other"][0]
        assert abs(logp[0] - exp_t) <= 1e-12
        assert abs(logp[1] - exp_o) <= 1e-12
        assert abs(lse[0] - (alpha + math.log1p((V - 1) * math.exp(-alpha)))) <= 1e-12


# -- P3: probabilities over all targets sum to one ------------------------------

def test_p3_brute_force_all_targets_sum_to_one(orc):
    inp = synth.config("tiny")
    rows = np.arange(8)
    V = inp.V
    h = np.repeat(inp.h[rows], V, axis=0)
    y = np.tile(np.arange(V, dtype=np.int32), len(rows))
    logp, lse = orc.forward(h, inp.W, y)
    tot = np.exp(logp.reshape(len(rows), V)).sum(axis=1)
    assert np.all(np.abs(tot - 1.0) <= 1e-12)
    lse = lse.reshape(len(rows), V)
    assert np.all(np.abs(lse - lse[:, :1]) <= 1e-12)


# -- P4: library log-softmax on materialised logits --------------------------

def test_p4_matches_library_log_softmax(orc):
    inp = synth.config("tiny")
    h = synth.bf16_bits_to_f32(inp.h).astype(np.float64)
    W = synth.bf16_bits_to_f32(inp.W).astype(np.float64)
    ls = scipy.special.log_softmax(h @ W.T, axis=1)
    want = ls[np.arange(inp.T), inp.y]
    want_lse = scipy.special.logsumexp(h @ W.T, axis=1)
    logp, lse = orc.forward(inp.h, inp.W, inp.y, vocab_block=1000)
    assert np.max(np.abs(logp - want)) <= 1e-12
    assert np.max(np.abs(lse - want_lse)) <= 1e-12


def test_p4_vocab_block_does_not_matter(orc):
    inp = synth.make_inputs(40, 64, 3001, 0.1)
    a = orc.forward(inp.h, inp.W, inp.y, vocab_block=8192)
    b = orc.forward(inp.h, inp.W, inp.y, vocab_block=97)
    assert np.max(np.abs(a[0] - b[0])) <= 1e-12


# -- P5: range partials and their merge ---------------------------------------------

@pytest.mark.parametrize("cuts", [[2048], [1000, 3500], [128, 256, 2048, 4000]])
def test_p5_merge_of_ranges_equals_unsharded(cuts, orc):
    inp = synth.make_inputs(48, 128, 4096, 0.15)
    # targets on both sides of every cut, so range ownership is exercised
    for i, c in enumerate(cuts):
        inp.y[2 * i], inp.y[2 * i + 1] = c - 1, c
    bounds = [0] + cuts + [inp.V]
    parts = [orc.partial(inp.h, inp.W[a:b], inp.y, a) for a, b in zip(bounds[:-1], bounds[1:])]
    owners = np.stack([p["owned"] for p in parts]).sum(axis=0)
    act = inp.y != -100
    assert np.all(owners[act] == 1) and np.all(owners[~act] == 0)
    logp, lse = orc.merge(parts, inp.y)
    ref_logp, ref_lse = orc.forward(inp.h, inp.W, inp.y)
    assert np.max(np.abs(logp - ref_logp)) <= 1e-12
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_p5_partial_statistics_closed_form(orc):
    # zero inputs: every logit is 0, so each range has m = 0 and s = its width
    h = np.zeros((3, 32), np.uint16)
    W = np.zeros((1000, 32), np.uint16)
    y = np.array([5, 700, -100], np.int32)
    p = orc.partial(h, W[300:1000], y, 300)
    assert list(p["m"][:2]) == [0.0, 0.0] and list(p["s"][:2]) == [700.0, 700.0]
    assert list(p["owned"]) == [False, True, False]
    assert p["m"][2] == -np.inf and p["s"][2] == 0.0


# -- P6: gradients -------------------------------------------------------------------

def _loss(orc, h, W, y, g):
    logp, _ = orc.forward(h, W, y)
    return float(np.dot(g, logp))


def test_p6_finite_differences(orc):
    inp = synth.make_inputs(12, 16, 50, 0.2)
    h = synth.bf16_bits_to_f32(inp.h).astype(np.float64)
    W = synth.bf16_bits_to_f32(inp.W).astype(np.float64) * 4.0
    g = inp.g.astype(np.float64)
    gh, gW = orc.backward(h, W, inp.y, g)
    rng = np.random.Generator(np.random.PCG64(11))
    eps = 1e-6
    for _ in range(32):
        t, k = rng.integers(0, h.shape[0]), rng.integers(0, h.shape[1])
        hp, hm = h.copy(), h.copy()
        hp[t, k] += eps
        hm[t, k] -= eps
        fd = (_loss(orc, hp, W, inp.y, g) - _loss(orc, hm, W, inp.y, g)) / (2 * eps)
        assert abs(fd - gh[t, k]) <= 1e-6 * max(1.0, abs(fd))
        v, k = rng.integers(0, W.shape[0]), rng.integers(0, W.shape[1])
        Wp, Wm = W.copy(), W.copy()
        Wp[v, k] += eps
        Wm[v, k] -= eps
        fd = (_loss(orc, h, Wp, inp.y, g) - _loss(orc, h, Wm, inp.y, g)) / (2 * eps)
        assert abs(fd - gW[v, k]) <= 1e-6 * max(1.0, abs(fd))


def test_p6_grad_W_columns_sum_to_zero(orc):
    inp = synth.make_inputs(30, 64, 700, 0.1)
    _, gW = orc.backward(inp.h, inp.W, inp.y, inp.g)
    assert np.max(np.abs(gW.sum(axis=0))) <= 1e-10 * np.linalg.norm(gW)


def test_p6_zero_weight_closed_form(orc):
    inp = synth.make_inputs(20, 32, 300, 0.2)
    W = np.zeros((inp.V, inp.H), np.uint16)
    gh, gW = orc.backward(inp.h, W, inp.y, inp.g)
    assert np.all(gh == 0.0)
    h = synth.bf16_bits_to_f32(inp.h).astype(np.float64)
    act = inp.y != -100
    want = np.zeros((inp.V, inp.H))
    for t in np.nonzero(act)[0]:
        coeff = -np.full(inp.V, 1.0 / inp.V)
        coeff[inp.y[t]] += 1.0
        want += inp.g[t] * np.outer(coeff, h[t])
    assert np.max(np.abs(gW - want)) <= 1e-12


def test_backward_row_and_vocab_restrictions(orc):
    inp = synth.make_inputs(25, 64, 900, 0.2)
    gh, gW = orc.backward(inp.h, inp.W, inp.y, inp.g)
    rows = [0, 3, 24, 7]
    assert np.max(np.abs(orc.backward_rows(inp.h, inp.W, inp.y, inp.g, rows) - gh[rows])) <= 1e-12
    vr = [0, 5, 899, int(inp.y[2]), 450]
    assert np.max(np.abs(orc.grad_W_rows(inp.h, inp.W, inp.y, inp.g, vr) - gW[vr])) <= 1e-12


# -- P7: masking -------------------------------------------------------------------

def test_p7_masked_rows(orc):
    inp = synth.make_inputs(40, 32, 500, 0.25)
    act = inp.y != -100
    assert (~act).sum() == 10
    logp, lse = orc.forward(inp.h, inp.W, inp.y)
    assert np.all(logp[~act] == 0.0) and np.all(lse[~act] == 0.0)
    assert not np.any(np.signbit(logp[~act]))
    gh, gW = orc.backward(inp.h, inp.W, inp.y, inp.g)
    assert np.all(gh[~act] == 0.0)
    gh2, gW2 = orc.backward(inp.h[act], inp.W, inp.y[act], inp.g[act])
    assert np.max(np.abs(gW - gW2)) <= 1e-13
    l2, _ = orc.forward(inp.h[act], inp.W, inp.y[act])
    assert np.max(np.abs(logp[act] - l2)) <= 1e-13


def test_out_of_range_target_raises(orc):
    inp = synth.make_inputs(4, 32, 100, 0.0)
    y = inp.y.copy()
    y[1] = 100
    with pytest.raises(ValueError):
        orc.forward(inp.h, inp.W, y)
    y[1] = -1
    with pytest.raises(ValueError):
        orc.forward(inp.h, inp.W, y)


# -- P8: row permutation -----------------------------------------------------------

def test_p8_row_permutation_equivariance(orc):
    inp = synth.make_inputs(37, 64, 1500, 0.15)
    perm = np.random.Generator(np.random.PCG64(9)).permutation(inp.T)
    a, _ = orc.forward(inp.h, inp.W, inp.y)
    b, _ = orc.forward(inp.h[perm], inp.W, inp.y[perm])
    assert np.max(np.abs(a[perm] - b)) <= 1e-13
