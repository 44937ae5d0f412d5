"""Pins of the oracle's RMSNorm: values worked by hand, closed forms and
invariants chosen so that a sum in place of the mean, a gain of w in place
of (1 + w), or eps outside the square root each fail."""
import numpy as np

from oracle import norm as N


def test_hand_worked_values():
    # x = (3, 4): mean of squares 12.5, rms = sqrt(12.5) = 3.5355339059327378
    y = N.rmsnorm([3.0, 4.0], eps=0.0)
    assert np.allclose(y, [0.8485281374238571, 1.1313708498984762], rtol=0, atol=1e-15)
    # zero-centred gain: (1 + 1.0) and (1 - 0.5)
    y = N.rmsnorm([3.0, 4.0], w=[1.0, -0.5], eps=0.0)
    assert np.allclose(y, [1.6970562748477142, 0.5656854249492381], rtol=0, atol=1e-15)


def test_eps_inside_the_root():
    # a constant row c with eps: c / sqrt(c^2 + eps); c = 1, eps = 3 -> 1/2
    y = N.rmsnorm(np.ones(8), eps=3.0)
    assert np.allclose(y, 0.5, rtol=0, atol=1e-15)
    assert np.array_equal(N.rmsnorm(np.zeros(16), eps=1e-5), np.zeros(16))


def test_invariants():
    r = np.random.default_rng(1)
    x = r.standard_normal((5, 4096)) * 3.0
    y = N.rmsnorm(x, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)     # unit rms
    assert np.allclose(N.rmsnorm(7.5 * x, eps=0.0), y, rtol=1e-14)          # scale invariance
    assert np.array_equal(N.rmsnorm(-x, eps=0.0), -y)                       # odd
    w = r.standard_normal(4096) * 0.1
    assert np.allclose(N.rmsnorm(x, w, eps=0.0), y * (1 + w), rtol=1e-15)   # rows independent
    assert np.allclose(N.rmsnorm(x[2:3], eps=0.0), y[2:3], rtol=0, atol=0)
