"""Pins of the oracle's quantizer and calibration against definitions computed independently
(exact rationals, brute force). CPU only."""
from fractions import Fraction
import itertools
import math

import numpy as np
import pytest

import oracle
import qssm_synth as synth


def rne_fraction(r: Fraction) -> int:
    """Round-half-to-even of an exact rational."""
    f = math.floor(r)
    rem = r - f
    if rem > Fraction(1, 2):
        return f + 1
    if rem < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def exact_code(v, s, lo=-128, hi=127):
    v = float(v)
    s = float(s)
    if not (2.0 ** -100 <= s <= 2.0 ** 100):
        return 0
    if math.isnan(v):
        return 0
    if math.isinf(v):
        return hi if v > 0 else lo
    q = rne_fraction(Fraction(v) / Fraction(s))
    return max(lo, min(hi, q))


SCALES = [np.float32(0.0371), np.float32(1.0), np.float32(3.0) / np.float32(7.0),
          np.float32(1e-3), np.float32(2.0 ** -20) * np.float32(3)]


@pytest.mark.parametrize("s", SCALES)
def test_quant_code_matches_exact_rational_rne(s):
    v = synth.quantizer_edge_values(scale=s, n=1500)
    got = oracle.quant_code(v, s)
    want = np.array([exact_code(a, s) for a in v], dtype=np.int8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_quant_code_random_scales_near_ties():
    r = np.random.default_rng(11)
    s = (r.uniform(0.5, 2.0, 3000) * 10.0 ** r.integers(-6, 4, 3000)).astype(np.float32)
    k = r.integers(-130, 130, 3000)
    v = ((k + 0.5) * s.astype(np.float64)).astype(np.float32)
    v = np.where(r.random(3000) < 0.5, v, np.nextafter(v, np.float32(np.inf) * np.sign(r.standard_normal(3000))).astype(np.float32))
    got = oracle.quant_code(v, s)
    want = np.array([exact_code(a, b) for a, b in zip(v, s)], dtype=np.int8)
    assert np.array_equal(got, want)


def test_quant_exact_ties_go_to_even():
    s = np.float32(0.5)
    v = np.array([0.25, 0.75, -0.25, -0.75, 1.25, 63.75, -64.25], dtype=np.float32)  # v/s = k + 1/2
    assert oracle.quant_code(v, s).tolist() == [0, 2, 0, -2, 2, 128 - 1, -128]


def test_quant_saturation_nan_inf_zero():
    s = np.float32(1.0)
    v = np.array([127.4, 127.5, 127.6, 1e9, -128.4, -128.5, -128.6, -1e9, np.inf, -np.inf, np.nan,
                  -0.0, 0.0], dtype=np.float32)
    assert oracle.quant_code(v, s).tolist() == [127, 127, 127, 127, -128, -128, -128, -128, 127,
                                                -128, 0, 0, 0]


@pytest.mark.parametrize("s", [0.0, -1.0, np.nan, np.inf, 2.0 ** -101, 2.0 ** 101])
def test_invalid_scale_gives_zero_codes(s):
    v = np.array([1.0, -5.0, 1e-30, 1e30], dtype=np.float32)
    assert oracle.quant_code(v, np.float32(s)).tolist() == [0, 0, 0, 0]


def test_scale_range_endpoints_valid():
    assert oracle.quant_code(np.float32(2.0 ** -100 * 3), np.float32(2.0 ** -100)) == 3
    assert oracle.quant_code(np.float32(2.0 ** 100 * -7), np.float32(2.0 ** 100)) == -7


def test_quant_group_x_layout_perm_and_groups():
    r = np.random.default_rng(3)
    outer, C, inner, G = 3, 7, 5, 3
    x = (r.standard_normal((outer, C, inner)) * 4).astype(np.float32)
    perm = r.permutation(C).astype(np.int32)
    group_of = r.integers(0, G, C).astype(np.uint8)
    scales = np.array([0.05, 0.11, 0.3], dtype=np.float32)
    q = oracle.quant_group_x(x, group_of, scales, perm=perm)
    for o, c, i in itertools.product(range(outer), range(C), range(inner)):
        assert q[o, c, i] == exact_code(x[o, perm[c], i], scales[group_of[c]])
    q0 = oracle.quant_group_x(x, group_of, scales)
    for o, c, i in itertools.product(range(outer), range(C), range(inner)):
        assert q0[o, c, i] == exact_code(x[o, c, i], scales[group_of[c]])


def test_quant_state_group_layout():
    r = np.random.default_rng(4)
    outer, Gbc, N, inner, gs = 2, 3, 8, 4, 4
    bc = (r.standard_normal((outer, Gbc, N, inner)) * 3).astype(np.float32)
    scales = r.uniform(0.01, 0.1, Gbc * N // gs).astype(np.float32)
    q = oracle.quant_state_group(bc, gs, scales)
    for o, g, n, i in itertools.product(range(outer), range(Gbc), range(N), range(inner)):
        assert q[o, g, n, i] == exact_code(bc[o, g, n, i], scales[g * (N // gs) + n // gs])


def nearest_f32(r: Fraction):
    """The fp32 numbers adjacent to the exact rational r, for a correct-rounding check."""
    f = np.float32(float(r))
    return f, np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))


def test_scale_from_absmax_is_correctly_rounded_and_clamped():
    r = np.random.default_rng(5)
    a = (r.uniform(0.5, 2, 500) * 10.0 ** r.integers(-20, 20, 500)).astype(np.float32)
    s = oracle.scale_from_absmax(a)
    for ai, si in zip(a, s):
        exact = Fraction(float(ai)) / 127
        err = abs(Fraction(float(si)) - exact)
        for nb in nearest_f32(exact)[1:]:
            assert err <= abs(Fraction(float(nb)) - exact)
    assert oracle.scale_from_absmax(np.float32(0.0)) == 1.0
    assert oracle.scale_from_absmax(np.float32(1e-35)) == np.float32(2.0 ** -100)
    assert oracle.scale_from_absmax(np.float32(3e38)) == np.float32(2.0 ** 100)


def test_group_scales_absmax_per_group():
    x = np.zeros((2, 4, 3), dtype=np.float32)
    x[1, 0, 2] = -12.7
    x[0, 2, 1] = 2.54
    x[0, 3, 0] = np.nan
    x[1, 3, 1] = np.inf
    x[0, 3, 2] = 0.5
    group_of = np.array([0, 1, 0, 1], dtype=np.uint8)
    s = oracle.group_scales(x, group_of, 2)
    assert s[0] == np.float32(12.7) / np.float32(127)
    assert s[1] == np.float32(0.5) / np.float32(127)  # NaN and Inf are ignored


def test_state_group_scales_contiguous_groups():
    bc = np.zeros((1, 2, 8, 2), dtype=np.float32)
    bc[0, 1, 5, 1] = 254.0    # group 1, state-group 1 (states 4..7)
    bc[0, 0, 3, 0] = -1.27    # group 0, state-group 0
    s = oracle.state_group_scales(bc, 4)
    assert s.tolist() == [np.float32(1.27) / np.float32(127), 1.0, 1.0, 2.0]
