"""Pins of the oracle's float32 RMSNorm.

Values worked by hand in float32 (exact rationals rounded once by the IEEE
rules), rows built so that each step of the fixed summation order decides
the result (a different order gives a different float32 sum, worked out
below), the float64 error bound of the whole chain, and invariants, chosen
so that a sum in place of the mean, a gain of w in place of (1 + w), eps
outside the square root, a multiplication by a rounded reciprocal in place
of the division, or a changed summation order each fail."""
import numpy as np
import pytest

from oracle import norm as N

F32 = np.float32


def _row(H, entries):
    x = np.zeros(H, np.float32)
    for i, v in entries.items():
        x[i] = v
    return x


def test_hand_worked_values():
    # x = (3, 4, 0, 0): sum of squares 25, mean 6.25, rms 2.5 (all exact);
    # 3 / 2.5 = 1.2 and 4 / 2.5 = 1.6 rounded to float32
    y = N.rmsnorm([3.0, 4.0, 0.0, 0.0], eps=0.0)
    assert y.dtype == np.float32
    assert y.tolist() == [float(F32(1.2)), float(F32(1.6)), 0.0, 0.0]
    assert float(y[0]) == 1.2000000476837158 and float(y[1]) == 1.600000023841858
    # zero-centred gain: 1.2 * (1 + 1) = 2.4 exactly twice the rounded 1.2;
    # (1 - 0.5) halves 1.6
    y = N.rmsnorm([3.0, 4.0, 0.0, 0.0], w=[1.0, -0.5, 0.0, 0.0], eps=0.0)
    assert y.tolist() == [2 * float(F32(1.2)), float(F32(1.6)) / 2, 0.0, 0.0]


def test_eps_inside_the_root():
    # a constant row c with eps: c / sqrt(c^2 + eps); c = 1, eps = 3 -> 1/2
    assert N.rmsnorm(np.ones(8), eps=3.0).tolist() == [0.5] * 8
    assert np.array_equal(N.rmsnorm(np.zeros(16), eps=1e-5), np.zeros(16))


def test_division_not_reciprocal():
    # x = (5, 1, 1, 3): sum of squares 36, mean 9, rms 3 (exact). 5 / 3
    # rounds to 1.6666666269302368; multiplying by the rounded reciprocal
    # would give 5 * 0.3333333432674408 = 1.66666671633..., which rounds up
    # to 1.6666667461395264.
    y = N.rmsnorm([5.0, 1.0, 1.0, 3.0], eps=0.0)
    assert y.tolist() == [1.6666666269302368, float(F32(1 / 3)), float(F32(1 / 3)), 1.0]
    assert float(F32(5) * (F32(1) / F32(3))) == 1.6666667461395264


def test_order_within_a_partial():
    # H = 1024: partial 0 holds columns 0..3 only. 4096^2 = 2^24, then three
    # squares of 1 added one at a time: 2^24 + 1 is a tie between 2^24 and
    # 2^24 + 2 and goes to the even 2^24, three times, so the sum is 2^24
    # (adding the three ones first would give 3 + 2^24 -> 2^24 + 4; a tree
    # (2^24 + 1) + (1 + 1) gives 2^24 + 2). Mean 2^24 / 1024 = 2^14, rms 2^7,
    # x0 / rms = 32 exactly; with 2^24 + 4 it would be 32 - 2^-18.
    x = _row(1024, {0: 4096.0, 1: 1.0, 2: 1.0, 3: 1.0})
    assert float(N.sum_of_squares(x)) == 2.0 ** 24
    y = N.rmsnorm(x, eps=0.0)
    assert float(y[0]) == 32.0 and float(y[1]) == 2.0 ** -7
    # the same four values in reverse column order: 1 + 1 + 1 = 3 first
    xr = _row(1024, {0: 1.0, 1: 1.0, 2: 1.0, 3: 4096.0})
    assert float(N.sum_of_squares(xr)) == 2.0 ** 24 + 4
    assert float(N.rmsnorm(xr, eps=0.0)[3]) == 32.0 - 2.0 ** -18


def test_order_across_column_blocks():
    # H = 2048: partial 5 holds columns 20..23 and 1044..1047, in that order.
    # 1 then 4096^2: 1 + 2^24 ties to 2^24 (1 lost). Reversed placement keeps
    # the same sum here, so put two ones first: 1 + 1 = 2, 2 + 2^24 exact.
    x = _row(2048, {20: 1.0, 21: 1.0, 1044: 4096.0})
    assert float(N.sum_of_squares(x)) == 2.0 ** 24 + 2
    x = _row(2048, {20: 4096.0, 1044: 1.0, 1045: 1.0})
    assert float(N.sum_of_squares(x)) == 2.0 ** 24            # each 1 lost in turn


def test_order_of_the_halving_fold():
    # partials 0, 16, 32, 48 of run 0 hold 2^24, 1, 1, 1 (columns 0, 64, 128,
    # 192). Fold m = 32: p0 = 2^24 + p32 = 2^24 + 1 -> 2^24 (tie to even),
    # p16 = p16 + p48 = 2. Fold m = 16: p0 = 2^24 + 2 (exact). A sequential
    # sum over p0, p1, ... would lose all three ones: 2^24.
    x = _row(1024, {0: 4096.0, 64: 1.0, 128: 1.0, 192: 1.0})
    assert float(N.sum_of_squares(x)) == 2.0 ** 24 + 2
    # partials 0 and 1: fold m = 1 is the last, so 2^24 + 1 -> 2^24 only
    # after the ones of partials 2 and 3 joined partial 0 and 1 first:
    # m = 2: p0 = 2^24 + p2 (1) -> 2^24, p1 = 1 + p3 (1) = 2; m = 1: 2^24 + 2
    x = _row(1024, {0: 4096.0, 4: 1.0, 8: 1.0, 12: 1.0})
    assert float(N.sum_of_squares(x)) == 2.0 ** 24 + 2


def test_order_of_the_run_sums():
    # runs 0..3 start at columns 0, 256, 512, 768: sums 2^24, 1, 1, 1 added
    # left to right: each 1 ties to even and is lost -> 2^24; pairwise
    # (2^24 + 1) + (1 + 1) would give 2^24 + 2
    x = _row(1024, {0: 4096.0, 256: 1.0, 512: 1.0, 768: 1.0})
    assert float(N.sum_of_squares(x)) == 2.0 ** 24
    # ((1 + 1) + 2^24) + 1: 2^24 + 2 is exact, then 2^24 + 3 is a tie between
    # 2^24 + 2 (odd last mantissa bit) and 2^24 + 4 (even): 2^24 + 4
    x = _row(1024, {0: 1.0, 256: 1.0, 512: 4096.0, 768: 1.0})
    assert float(N.sum_of_squares(x)) == 2.0 ** 24 + 4


def test_squares_rounded_before_the_sum():
    # 1 + 2^-12: its square 1 + 2^-11 + 2^-24 rounds to 1 + 2^-11 in float32;
    # the row (a, a, 0, 0) then sums to 2 + 2^-10 exactly
    a = F32(1.0 + 2.0 ** -12)
    x = np.array([a, a, 0, 0], np.float32)
    assert float(N.sum_of_squares(x)) == 2.0 + 2.0 ** -10


@pytest.mark.parametrize("H", [4, 12, 256, 1000, 4096, 8192])
def test_error_bound_against_float64(H):
    """The float32 chain against the exact value (float64 is exact for the
    squares and within 2^-53 H for the sum): the sum's error is at most
    (n_seq + 8) u sum(x^2) with n_seq the additions of one partial and u =
    2^-24, the mean and root add u each, the quotient and gain product u
    each; 24 ulp of slack covers every H here."""
    g = np.random.default_rng(H)
    x = (g.standard_normal((7, H)) * np.exp(g.uniform(-20, 20, (7, 1)))).astype(np.float32)
    w = (g.standard_normal(H) * 0.1).astype(np.float32)
    x64, w64 = x.astype(np.float64), w.astype(np.float64)
    ss64 = np.sum(x64 * x64, axis=1)
    n_seq = 4 * ((H + 1023) // 1024)
    bound = (n_seq + 8) * 2.0 ** -24 * ss64
    assert np.all(np.abs(N.sum_of_squares(x).astype(np.float64) - ss64) <= bound)
    y64 = x64 / np.sqrt(ss64 / H + 1e-5)[:, None] * (1.0 + w64)
    y = N.rmsnorm(x, w, eps=1e-5).astype(np.float64)
    tol = (n_seq + 24) * 2.0 ** -24 * np.abs(y64) + 1e-300
    assert np.all(np.abs(y - y64) <= tol)


def test_invariants():
    r = np.random.default_rng(1)
    x = (r.standard_normal((5, 4096)) * 3.0).astype(np.float32)
    y = N.rmsnorm(x, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y.astype(np.float64) ** 2, axis=1)), 1.0, rtol=1e-6)
    # a power of two scales every step exactly (no eps): same result
    assert np.array_equal(N.rmsnorm(np.float32(8.0) * x, eps=0.0), y)
    assert np.array_equal(N.rmsnorm(-x, eps=0.0), -y)                 # odd
    assert np.array_equal(N.rmsnorm(x[2:3], eps=0.0), y[2:3])          # rows independent
    w = (r.standard_normal(4096) * 0.1).astype(np.float32)
    assert np.array_equal(N.rmsnorm(x, w, eps=0.0), y * (np.float32(1) + w))
