"""Pins of the RL-objective oracle (oracle/rl_loss.py) to closed forms and
to finite differences (not to its own formula).

P-R1 on-policy tokens (logp = logp_old): r = 1, loss = -A, g = -A.
P-R2 clipped regions: A > 0 with r above 1 + eps_high gives loss
     -(1 + eps_high) A and g = 0; A < 0 with r below 1 - eps_low gives
     loss -(1 - eps_low) A and g = 0.
P-R3 the k3 term: zero when logp_ref = logp; its value at d = ln 2 is
     2 - ln 2 - 1; always >= 0.
P-R4 g equals a central finite difference of the loss in logp (fp64, away
     from the clip kinks), with and without the KL term.
P-R5 ignored rows: loss = g = 0; scale multiplies both.
"""
import math

import numpy as np

from oracle import rl_loss as orl


def test_on_policy_closed_form():
    A = np.array([-2.0, -0.5, 0.0, 0.75, 3.0])
    lp = np.array([-1.0, -3.0, -0.1, -7.0, -2.5])
    loss, g = orl.token_loss(lp, lp, A, np.zeros(5, dtype=np.int32), 0.2, 0.28)
    assert np.array_equal(loss, -A)
    assert np.array_equal(g, -A)


def test_clipped_regions():
    eps_lo, eps_hi = 0.2, 0.28
    # A > 0, r = e^0.5 > 1.28: clipped above
    loss, g = orl.token_loss([-1.0], [-1.5], [2.0], [0], eps_lo, eps_hi)
    assert math.isclose(loss[0], -(1 + eps_hi) * 2.0, rel_tol=1e-15) and g[0] == 0.0
    # A < 0, r = e^-0.5 < 0.8: clipped below
    loss, g = orl.token_loss([-1.5], [-1.0], [-3.0], [0], eps_lo, eps_hi)
    assert math.isclose(loss[0], (1 - eps_lo) * 3.0, rel_tol=1e-15) and g[0] == 0.0
    # A > 0, r below the range: the unclipped term is smaller, gradient flows
    loss, g = orl.token_loss([-1.5], [-1.0], [2.0], [0], eps_lo, eps_hi)
    r = math.exp(-0.5)
    assert math.isclose(loss[0], -r * 2.0, rel_tol=1e-15) and math.isclose(g[0], -r * 2.0, rel_tol=1e-15)


def test_k3_closed_forms():
    lp = np.array([-2.0, -2.0])
    ref = np.array([-2.0, -2.0 + math.log(2.0)])
    loss, g = orl.token_loss(lp, lp, np.zeros(2), [0, 0], 0.2, 0.2, beta=1.0, logp_ref=ref)
    assert loss[0] == 0.0 and g[0] == 0.0
    assert math.isclose(loss[1], 2.0 - math.log(2.0) - 1.0, rel_tol=1e-14)
    assert math.isclose(g[1], 1.0 - 2.0, rel_tol=1e-14)
    gen = np.random.Generator(np.random.PCG64(3))
    d = gen.normal(0, 2, 1000)
    loss, _ = orl.token_loss(np.zeros(1000), np.zeros(1000), np.zeros(1000), np.zeros(1000), 0.2, 0.2,
                             beta=1.0, logp_ref=d)
    assert np.all(loss >= 0.0)


def test_gradient_finite_differences():
    gen = np.random.Generator(np.random.PCG64(4))
    n = 400
    lp = -gen.uniform(0.1, 8.0, n)
    old = lp + gen.normal(0, 0.3, n)
    A = gen.normal(0, 1, n)
    ref = lp + gen.normal(0, 0.2, n)
    y = np.zeros(n, dtype=np.int32)
    eps_lo, eps_hi, beta = 0.2, 0.28, 0.05
    r = np.exp(lp - old)
    away = (np.abs(r - (1 - eps_lo)) > 1e-3) & (np.abs(r - (1 + eps_hi)) > 1e-3)
    h = 1e-6
    for b in (0.0, beta):
        _, g = orl.token_loss(lp, old, A, y, eps_lo, eps_hi, beta=b, logp_ref=ref)
        lp_hi, _ = orl.token_loss(lp + h, old, A, y, eps_lo, eps_hi, beta=b, logp_ref=ref)
        lp_lo, _ = orl.token_loss(lp - h, old, A, y, eps_lo, eps_hi, beta=b, logp_ref=ref)
        fd = (lp_hi - lp_lo) / (2 * h)
        assert np.all(np.abs(fd - g)[away] <= 1e-6 * (1 + np.abs(g[away])))


def test_ignored_rows_and_scale():
    lp = np.array([-1.0, -2.0, -3.0])
    old = np.array([-1.1, -2.0, -2.5])
    A = np.array([1.0, -1.0, 0.5])
    y = np.array([5, -100, 7], dtype=np.int32)
    loss1, g1 = orl.token_loss(lp, old, A, y, 0.2, 0.2)
    loss2, g2 = orl.token_loss(lp, old, A, y, 0.2, 0.2, scale=0.25)
    assert loss1[1] == 0.0 and g1[1] == 0.0
    assert np.array_equal(loss2, 0.25 * loss1) and np.array_equal(g2, 0.25 * g1)
