"""Pins of the oracle's soft-edge code: the page's byte layout (golden table), an exact-rational
brute force of the encoder, special values, the threshold rule and the mode shares. CPU only."""
from fractions import Fraction
import math
import os

import numpy as np
import pytest

import oracle
from tests.test_oracle_quant import rne_fraction

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_layout(name="softedge_layout.txt"):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b, mode, lo, hi, mult = line.split()
        rows.append((int(a, 16), int(b, 16), mode, int(lo), int(hi), Fraction(mult)))
    return rows


def load_thresholds():
    d = {}
    for line in open(os.path.join(GOLDEN, "softedge_thresholds.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            d[k] = float(v)
    return d


LAYOUTS = {4: "softedge_layout.txt", 2: "softedge_layout_shift.txt"}


@pytest.mark.parametrize("ratio", [4, 2])
@pytest.mark.parametrize("s", [np.float32(1.0), np.float32(0.0173), np.float32(2.0 ** -90)])
def test_decode_table_matches_page_layout(s, ratio):
    table = oracle.softedge_value_table(s, ratio)
    covered = 0
    for a, b, mode, lo, hi, mult in load_layout(LAYOUTS[ratio]):
        assert b - a == hi - lo
        for k, byte in enumerate(range(a, b + 1)):
            want = Fraction(lo + k) * mult * Fraction(float(s))
            assert Fraction(float(table[byte])) == want, (hex(byte), mode)
            covered += 1
    assert covered == 256


def exact_softedge(v, s, L, H, ratio=4):
    v, s, L, H = float(v), float(s), float(L), float(H)
    if not (2.0 ** -100 <= s <= 2.0 ** 100) or math.isnan(v):
        return 0
    a = abs(v)
    small, large = a < L, a > H
    if small and not large:
        base, lo, hi, tag, mask = Fraction(s) / ratio, -32, 31, 0x80, 0x3F
    elif large and not small:
        base, lo, hi, tag, mask = Fraction(s) * ratio, -32, 31, 0xC0, 0x3F
    else:
        base, lo, hi, tag, mask = Fraction(s), -64, 63, 0x00, 0x7F
    if math.isinf(v):
        q = hi if v > 0 else lo
    else:
        q = max(lo, min(hi, rne_fraction(Fraction(v) / base)))
    return tag | (q & mask)


@pytest.mark.parametrize("ratio", [4, 2])
def test_encode_matches_exact_brute_force(ratio):
    r = np.random.default_rng(21)
    s, L, H = np.float32(0.05), np.float32(0.2), np.float32(3.1)
    ties = []
    for base, span in ((float(s) / ratio, 34), (float(s), 66), (float(s) * ratio, 34)):
        k = np.arange(-span, span) + 0.5
        t = (k * base).astype(np.float32)
        ties += [t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(-np.inf))]
    v = np.concatenate([
        (r.standard_normal(20000) * 1.5).astype(np.float32),
        (r.standard_normal(2000) * 20).astype(np.float32),
        *ties,
        np.array([L, -L, H, -H, np.nextafter(L, np.float32(0)), np.nextafter(H, np.float32(9)),
                  0.0, -0.0, np.inf, -np.inf, np.nan], dtype=np.float32),
    ]).astype(np.float32)
    got = oracle.softedge_encode(v.reshape(1, 1, -1), np.zeros(1, np.uint8), [s], [L], [H],
                                 ratio=ratio).ravel()
    want = np.array([exact_softedge(a, s, L, H, ratio) for a in v], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_special_values():
    s, L, H = np.float32(1.0), np.float32(0.5), np.float32(60.0)
    v = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, 0.3, 70.0, -70.0, 30.0], dtype=np.float32)
    c = oracle.softedge_encode(v.reshape(1, 1, -1), np.zeros(1, np.uint8), [s], [L], [H]).ravel()
    # NaN -> 0x00; +Inf -> large +31; -Inf -> large -32; -0 and 0 -> small 0; 0.3/(1/4) = 1.2 -> 1;
    # 70/4 = 17.5 -> 18 (even); -70/4 -> -18; 30 -> standard 30
    assert [hex(b) for b in c] == ["0x0", "0xdf", "0xe0", "0x80", "0x80", "0x81", "0xd2", "0xee",
                                   "0x1e"]
    # L = 0: nothing is small; L > H: both tests true -> the standard (default) case
    c2 = oracle.softedge_encode(np.array([[[0.0, 5.0]]], np.float32), np.zeros(1, np.uint8), [s],
                                [np.float32(0.0)], [H]).ravel()
    assert c2.tolist() == [0x00, 0x05]
    c3 = oracle.softedge_encode(np.array([[[3.0]]], np.float32), np.zeros(1, np.uint8), [s],
                                [np.float32(10.0)], [np.float32(1.0)]).ravel()
    assert c3.tolist() == [0x03]


def test_roundtrip_error_within_half_step():
    r = np.random.default_rng(5)
    s, L, H = np.float32(0.04), np.float32(0.1), np.float32(2.5)
    v = (r.standard_normal(50000)).astype(np.float32)
    c = oracle.softedge_encode(v.reshape(1, 1, -1), np.zeros(1, np.uint8), [s], [L], [H]).ravel()
    back = oracle.softedge_values(c.reshape(1, 1, -1), np.zeros(1, np.uint8), [s]).ravel()
    a = np.abs(v.astype(np.float64))
    step = np.where(a < L, float(s) / 4, np.where(a > H, 4 * float(s), float(s)))
    sat = np.where(a > H, 31.5 * 4 * float(s), np.inf)
    ok = (np.abs(back - v) <= step / 2 + 1e-12) | (a > sat)
    assert ok.all()


def test_percentile_rule_closed_form():
    # |v| = 0, 1, ..., 1000: linear-interpolation percentiles are exactly 50 and 999
    v = np.arange(1001, dtype=np.float32) * np.where(np.arange(1001) % 2, -1, 1).astype(np.float32)
    s, L, H, state = oracle.softedge_thresholds(v)
    t = load_thresholds()
    assert (oracle.SOFTEDGE_P_LOW, oracle.SOFTEDGE_P_HIGH, oracle.SOFTEDGE_EMA_ALPHA) == (
        t["p_low"], t["p_high"], t["ema_alpha"])
    assert (L, H) == (np.float32(50.0), np.float32(999.0))
    assert s == np.float32(999.0) / np.float32(63.0)
    # EMA with alpha = 0.1 against a hand-computed blend
    s2, L2, H2, _ = oracle.softedge_thresholds(v * 2, prev=state)
    assert L2 == np.float32(0.1 * 100.0 + 0.9 * 50.0)
    assert H2 == np.float32(0.1 * 1998.0 + 0.9 * 999.0)


def test_mode_shares_at_default_thresholds():
    """Section 2.1: the standard mode covers about 95% of typical activations. With L = P5 and
    H = P99.9 of the same sample the shares are 5% / 94.9% / 0.1% by construction."""
    r = np.random.default_rng(8)
    v = r.standard_normal(200001).astype(np.float32)
    s, L, H, _ = oracle.softedge_thresholds(v)
    c = oracle.softedge_encode(v.reshape(1, 1, -1), np.zeros(1, np.uint8), [s], [L], [H]).ravel()
    small = np.mean((c & 0xC0) == 0x80)
    large = np.mean((c & 0xC0) == 0xC0)
    std = np.mean((c & 0x80) == 0)
    assert abs(small - 0.05) < 1e-3 and abs(large - 0.001) < 2e-4
    assert abs(std - load_thresholds()["standard_share_approx"]) < 0.01


def test_invalid_base_scale_encodes_zero():
    v = np.array([[[1.0, -3.0, 100.0]]], np.float32)
    for s in (0.0, np.nan, -1.0, np.inf):
        c = oracle.softedge_encode(v, np.zeros(1, np.uint8), [np.float32(s)], [np.float32(0.5)],
                                   [np.float32(5.0)])
        assert c.ravel().tolist() == [0, 0, 0]


def test_shift_form_special_values():
    """Section 4.1 form (scale/2, scale*2): worked by hand for s = 1, L = 0.5, H = 60."""
    s, L, H = np.float32(1.0), np.float32(0.5), np.float32(60.0)
    v = np.array([np.inf, -np.inf, 0.3, 0.25, 70.0, -70.0, 61.0, 30.0], dtype=np.float32)
    c = oracle.softedge_encode(v.reshape(1, 1, -1), np.zeros(1, np.uint8), [s], [L], [H],
                               ratio=2).ravel()
    # +-Inf saturate in the large mode; 0.3 / 0.5 = 0.6 -> 1; 0.25 / 0.5 = 0.5 -> 0 (even);
    # 70 / 2 = 35 -> 31 (saturated); -70 / 2 -> -32; 61 / 2 = 30.5 -> 30 (even); 30 standard
    assert [hex(b) for b in c] == ["0xdf", "0xe0", "0x81", "0x80", "0xdf", "0xe0", "0xde", "0x1e"]
    # the two forms differ only in the mode scales: standard bytes decode alike
    t4 = oracle.softedge_value_table(np.float32(0.37), 4)
    t2 = oracle.softedge_value_table(np.float32(0.37), 2)
    assert np.array_equal(t4[:128], t2[:128])
    assert np.array_equal(t4[0x80:0xC0] * 2, t2[0x80:0xC0])
    assert np.array_equal(t4[0xC0:], t2[0xC0:] * 2)


def brute_percentile(vals, pct):
    """Linear-interpolation percentile by the textbook definition, with exact rationals: sorted
    values a_0 <= ... <= a_{n-1}, position (n - 1) p / 100, interpolation between its neighbours."""
    a = sorted(Fraction(abs(float(v))) for v in vals)
    pos = Fraction(len(a) - 1) * Fraction(pct) / 100
    k = int(pos)
    if k >= len(a) - 1:
        return a[-1]
    return a[k] + (a[k + 1] - a[k]) * (pos - k)


def test_track_groups_and_permutation_by_brute_force():
    """softedge_track gathers each group's values through the permutation: against group-wise
    exact-rational percentiles of hand-collected values on a tiny tensor. The tolerance is the fp64
    rounding of the interpolation position (0.999 is not a binary fraction): about 1e-13 relative
    here, far below the gap between neighbouring order statistics that a wrong rank would show."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((3, 6, 37)) * np.array([0.1, 5, 1, 30, 2, 0.5])[None, :, None])
    x = x.astype(np.float32)
    perm = np.array([3, 0, 5, 1, 4, 2], np.int32)
    group_of = np.array([0, 1, 1, 2, 0, 2], np.uint8)
    s, L, H, st = oracle.softedge_track(x, group_of, 3, perm=perm)
    for g in range(3):
        vals = [x[o, perm[c], i] for o in range(3) for c in range(6) if group_of[c] == g
                for i in range(37)]
        lw, hw = brute_percentile(vals, 5), brute_percentile(vals, Fraction(999, 10))
        assert abs(st[g][0] - float(lw)) <= 1e-12 * float(lw)
        assert abs(st[g][1] - float(hw)) <= 1e-12 * float(hw)
        assert H[g] == np.float32(st[g][1]) and s[g] == np.float32(H[g] / np.float32(63))


def test_track_ema_chain_and_empty_group():
    """Three batches: the state follows L_t = 0.1 P5_t + 0.9 L_{t-1} from the first batch's own
    percentiles; a group with no channels keeps its state."""
    v = [np.arange(1001, dtype=np.float32) * k for k in (1, 2, 4)]
    st = None
    lw = hw = None
    for k, vk in enumerate(v):
        s, L, H, st = oracle.softedge_track(vk.reshape(1, 1, -1), np.zeros(1, np.uint8), 2,
                                            prev=st)
        p5, p999 = 50.0 * (1, 2, 4)[k], 999.0 * (1, 2, 4)[k]
        lw = p5 if lw is None else 0.1 * p5 + 0.9 * lw
        hw = p999 if hw is None else 0.1 * p999 + 0.9 * hw
        # the fp64 position of P99.9 carries one rounding (0.999 is not a binary fraction)
        assert st[0][0] == lw and abs(st[0][1] - hw) <= 1e-13 * hw
        assert (L[0], H[0]) == (np.float32(lw), np.float32(hw))
        assert (L[1], H[1], s[1]) == (0, 0, 1) and st[1] == (0.0, 0.0)
