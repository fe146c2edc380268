"""Pins for the prologue oracle (oracle/prologue.py): closed forms and
identities that a dropped term, a wrong sign or a wrong clamp would break."""
from __future__ import annotations

import math

import numpy as np

from oracle import prologue as P


def test_sigmoid_values_and_symmetry():
    assert P.sigmoid(0.0) == 0.5
    assert abs(P.sigmoid(math.log(3.0)) - 0.75) < 1e-15          # 1 / (1 + 1/3)
    x = np.linspace(-40, 40, 161)
    np.testing.assert_allclose(P.sigmoid(x) + P.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    big = P.sigmoid(np.array([-1000.0, 1000.0]))                  # no overflow
    assert big[0] == 0.0 and big[1] == 1.0


def test_softplus_values_and_identity():
    assert abs(P.softplus(0.0) - math.log(2.0)) < 1e-16
    assert abs(P.softplus(math.log(math.e - 1.0)) - 1.0) < 1e-15   # log(1 + (e - 1)) = 1
    x = np.linspace(-50, 50, 201)
    np.testing.assert_allclose(P.softplus(x) - P.softplus(-x), x, rtol=0, atol=1e-12)
    assert P.softplus(1000.0) == 1000.0
    assert P.softplus(-1000.0) == 0.0


def test_log_decay_range_and_floor():
    x = np.linspace(-60, 60, 241)
    d = P.log_decay(x)
    assert np.all(d <= 0.0) and np.all(d >= P.G_MIN)
    assert np.all(np.diff(d) <= 0.0)                     # decreasing in x
    assert P.log_decay(10.0) == P.G_MIN                   # softplus(10) > 5: clamped
    assert abs(P.log_decay(0.0) + math.log(2.0)) < 1e-16
    # the floor bites exactly where softplus(x) = 5, at x = log(e^5 - 1)
    x5 = math.log(math.exp(5.0) - 1.0)
    assert abs(P.log_decay(x5 - 1e-6) - P.G_MIN) < 1e-5 and P.log_decay(x5 + 1e-6) == P.G_MIN


def test_l2norm_closed_form():
    x = np.zeros((2, 4))
    x[0, 0] = 3.0
    x[0, 2] = 4.0                                         # norm 5
    y = P.l2norm(x)
    np.testing.assert_allclose(y[0], x[0] / math.sqrt(25.0 + P.NORM_EPS), rtol=1e-15)
    np.testing.assert_array_equal(y[1], 0.0)             # zero vector stays zero
    r = np.random.default_rng(0).standard_normal((5, 3, 128)) * 7.0
    n = np.linalg.norm(P.l2norm(r), axis=-1)
    np.testing.assert_allclose(n, 1.0, rtol=0, atol=1e-8)
    # direction is kept: y is a positive multiple of x
    np.testing.assert_allclose(P.l2norm(r) * np.linalg.norm(r, axis=-1, keepdims=True), r,
                               rtol=1e-7)


def test_apply_respects_each_flag():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((3, 2, 8)), rng.standard_normal((3, 2, 8))
    beta, g = rng.standard_normal((3, 2)), rng.standard_normal((3, 2, 8))
    out = P.apply(q, k, beta, g, 0)
    for a, b in zip(out, (q, k, beta, g)):
        np.testing.assert_array_equal(a, b)
    q1, k1, b1, g1 = P.apply(q, k, beta, g, P.QK_L2NORM)
    nq = np.linalg.norm(q, axis=-1)
    np.testing.assert_allclose(np.linalg.norm(q1, axis=-1), nq / np.sqrt(nq * nq + P.NORM_EPS),
                               rtol=1e-14)
    np.testing.assert_array_equal(b1, beta)
    _, _, b2, g2 = P.apply(q, k, beta, g, P.BETA_SIGMOID | P.G_SOFTPLUS)
    np.testing.assert_allclose(b2, P.sigmoid(beta))
    np.testing.assert_allclose(g2, P.log_decay(g))
