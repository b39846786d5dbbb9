"""Pins of the oracle's W4A8 linear layer (Quamba2 abstract: W4A8 for large-batch decoding):
the 4-bit quantizer against exact rational rounding, the scale rule against an exact quotient,
and the GEMM against a brute-force sum of exact fractions. CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def rne_frac(v, s, lo, hi):
    """clamp(RNE(v / s), lo, hi) on exact rationals (NaN -> 0, +-inf saturate)."""
    if np.isnan(v):
        return 0
    if np.isinf(v):
        return hi if v > 0 else lo
    q = Fraction(float(v)) / Fraction(float(s))
    f = q.numerator // q.denominator
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return max(lo, min(hi, f))


def test_quant_w4_exact_rounding():
    r = np.random.default_rng(1)
    N, K, group = 6, 64, 16
    w = (r.standard_normal((N, K)) * np.exp(r.uniform(-3, 3, (N, 1)))).astype(np.float32)
    s = oracle.w4_scales(w, group)
    # exact ties and near-ties, saturation both ways, NaN and infinities
    w[0, :8] = (np.array([0.5, 1.5, 2.5, -0.5, -1.5, 7.5, -8.5, 3.5], np.float32) * s[0, 0])
    w[1, 0] = np.nextafter(np.float32(2.5) * s[1, 0], np.float32(10))
    w[1, 1] = np.nextafter(np.float32(2.5) * s[1, 0], np.float32(-10))
    w[2, 16:20] = [np.nan, np.inf, -np.inf, 1e30]
    s[3, 1] = np.float32(1e-35)  # invalid scale: the whole group encodes 0
    q = oracle.quant_w4(w, group, s)
    for n in range(N):
        for k in range(K):
            sc = s[n, k // group]
            want = 0 if not (2.0 ** -100 <= sc <= 2.0 ** 100) else rne_frac(w[n, k], sc, -8, 7)
            assert q[n, k] == want, (n, k, w[n, k], sc)
    assert q[0, :8].tolist() == [0, 2, 2, 0, -2, 7, -8, 4]
    assert not q[3, 16:32].any()


def test_w4_scale_rule():
    a = np.array([0.0, 7.0, 1.0, 3e-35, 1e35, 0.123456], np.float32)
    w = np.zeros((len(a), 8), np.float32)
    w[:, 3] = -a
    s = oracle.w4_scales(w, 8)[:, 0]
    for v, got in zip(a, s):
        want = 1.0 if v == 0 else float(np.clip(np.float32(Fraction(float(v)) / 7), 2.0 ** -100, 2.0 ** 100))
        assert got == np.float32(want)


def test_gemm_brute_force():
    r = np.random.default_rng(2)
    M, N, K, group = 3, 4, 32, 8
    qa = r.integers(-128, 128, (M, K)).astype(np.int8)
    qw = r.integers(-8, 8, (N, K)).astype(np.int8)
    sa = np.float32(0.0173)
    sw = np.exp(r.uniform(-4, 0, (N, K // group))).astype(np.float32)
    sw[2, 1] = np.float32(2.0 ** 101)  # invalid: that group contributes nothing
    bias = r.standard_normal(N)
    y = oracle.gemm_w4a8(qa, sa, qw, sw, group, bias)
    for m in range(M):
        for n in range(N):
            acc = Fraction(float(bias[n]))
            for k in range(K):
                s = sw[n, k // group]
                if not (2.0 ** -100 <= s <= 2.0 ** 100):
                    continue
                acc += Fraction(float(sa)) * Fraction(float(s)) * int(qa[m, k]) * int(qw[n, k])
            assert y[m, n] == pytest.approx(float(acc), rel=1e-14, abs=1e-14)


def test_gemm_groups_invariant_and_integer_case():
    """With unit scales and no bias the result is the integer matrix product exactly; with equal
    scales in every group, any group size gives the same result as one group per channel."""
    r = np.random.default_rng(3)
    M, N, K = 5, 7, 64
    qa = r.integers(-128, 128, (M, K)).astype(np.int8)
    qw = r.integers(-8, 8, (N, K)).astype(np.int8)
    y = oracle.gemm_w4a8(qa, 1.0, qw, np.ones((N, 1), np.float32), K)
    assert np.array_equal(y, qa.astype(np.int64) @ qw.astype(np.int64).T)
    sw = np.full((N, 1), 0.03125, np.float32)
    y1 = oracle.gemm_w4a8(qa, 0.5, qw, sw, K)
    for group in (8, 16, 32):
        y2 = oracle.gemm_w4a8(qa, 0.5, qw, np.repeat(sw, K // group, axis=1), group)
        assert np.array_equal(y1, y2)
