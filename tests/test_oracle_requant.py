"""Pins of the oracle's persistent-int8 output step (SSDi8 abstract: int8 activations handed to the
next W8A8 module, with an error-correction term from per-channel error statistics). The expected
codes below were worked out by hand from the int8 rule (exact quotient, round half to even,
saturation to [-128, 127], NaN to 0, an invalid scale to 0), with every operand a dyadic value
that fp32 holds exactly."""
from fractions import Fraction

import numpy as np

import oracle

NAN, INF = float("nan"), float("inf")


def test_requant_output_hand_table():
    # channel: group, then six values; scales per group: 0.5, 4, 1e-35 (invalid: below 2^-100)
    group_of = np.array([0, 1, 0, 2], np.uint8)
    scales = np.array([0.5, 4.0, 1e-35], np.float32)
    bias = np.array([0.0, 0.25, -0.125, 0.0], np.float32)
    y = np.array([[[0.25, 0.75, -0.25, 63.75, 100.0, NAN],        # /0.5
                   [1.75, 5.75, -2.25, -600.0, 9.0, INF],          # +0.25, /4
                   [0.375, 1.125, -0.125, 0.0, -64.125, -INF],     # -0.125, /0.5
                   [1.0, 2.0, -3.0, 1e30, -1e30, 0.5]]])           # invalid scale
    want = np.array([[[0, 2, 0, 127, 127, 0],
                      [0, 2, 0, -128, 2, 127],
                      [0, 2, 0, 0, -128, -128],
                      [0, 0, 0, 0, 0, 0]]], np.int8)
    got = oracle.requant_output(y, group_of, scales, bias)
    assert got.dtype == np.int8
    assert np.array_equal(got, want), got


def test_requant_output_decides_in_fp32():
    # y = 1 + 2^-30 is 1.0 in fp32: 1.0 / 2 is an exact tie and rounds to 0 (an fp64 decision
    # would see 0.5 + 2^-31 and give 1).
    y = np.array([[[1.0 + 2.0 ** -30]]])
    assert oracle.requant_output(y, [0], [2.0]) == 0
    # the bias is added in fp32: 2^24 + 1 rounds (tie to even) to 2^24, and 2^24 / 2^25 is a tie
    # that rounds to 0 (an exact sum would give 0.5 + 2^-25 and code 1)
    y = np.array([[[2.0 ** 24]]])
    assert oracle.requant_output(y, [0], [2.0 ** 25], bias=[1.0]) == 0
    assert oracle.requant_output(y, [0], [2.0 ** 25], bias=[2.0]) == 1


def test_requant_output_without_bias_is_the_plain_rule_per_group():
    """No bias: each channel's codes follow the exact-rational rule with its own group's scale
    (checked with Fractions on random fp32 values)."""
    rng = np.random.default_rng(5)
    C, inner = 6, 40
    group_of = rng.integers(0, 3, size=C).astype(np.uint8)
    scales = np.array([0.013, 0.2, 1.7], np.float32)
    y = (rng.standard_normal((2, C, inner)) * 2.0).astype(np.float32)
    got = oracle.requant_output(y, group_of, scales)
    for o in range(2):
        for c in range(C):
            s = Fraction(float(scales[group_of[c]]))
            for i in range(inner):
                r = Fraction(float(y[o, c, i])) / s
                k = r.numerator // r.denominator
                f = r - k
                q = k + (1 if f > Fraction(1, 2) or (f == Fraction(1, 2) and k % 2) else 0)
                assert got[o, c, i] == max(-128, min(127, q))


def test_channel_error_mean_closed_form():
    # ref = approx + c[d] + noise with noise in +-pairs along inner: the mean is c[d] exactly
    rng = np.random.default_rng(6)
    outer, C, inner = 3, 5, 8
    approx = rng.integers(-64, 64, size=(outer, C, inner)).astype(np.float64) / 16
    c = np.array([0.5, -0.25, 0.0, 1.0, -3.0])
    half = rng.integers(-32, 32, size=(outer, C, inner // 2)).astype(np.float64) / 8
    noise = np.concatenate([half, -half], axis=2)
    ref = approx + c[None, :, None] + noise
    assert np.array_equal(oracle.channel_error_mean(ref, approx), c)


def test_channel_error_mean_brute_force():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((2, 3, 4)).astype(np.float32)
    approx = rng.standard_normal((2, 3, 4)).astype(np.float32)
    got = oracle.channel_error_mean(ref, approx)
    for c in range(3):
        tot = sum(Fraction(float(ref[o, c, i])) - Fraction(float(approx[o, c, i]))
                  for o in range(2) for i in range(4))
        assert abs(got[c] - float(tot / 8)) <= 1e-15 * max(1.0, abs(float(tot / 8)))
