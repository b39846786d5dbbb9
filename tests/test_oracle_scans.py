"""Pins of the oracle's recurrences against closed forms, brute-force unrolled sums, a textbook
routine (matrix exponential, convolution) and invariants. CPU only."""
import itertools
import math

import numpy as np
import pytest
import scipy.linalg

import oracle
import qssm_synth as synth


# ------------------------------------------------------------------------------------------------
# Mamba1 selective scan

def small_m1(seed=0, B=2, L=7, D=3, N=4, Gbc=1, h0=True):
    r = np.random.default_rng(seed)
    return dict(
        xh=r.standard_normal((B, D, L)), delta=r.uniform(0.05, 0.9, (B, D, L)),
        A=-np.exp(r.uniform(-1, 1, (D, N))), Bh=r.standard_normal((B, Gbc, N, L)),
        Ch=r.standard_normal((B, Gbc, N, L)), Dskip=r.standard_normal(D),
        h0=r.standard_normal((B, D, N)) if h0 else None)


def unrolled_y(p):
    """y_t = sum_n [ C_t prod_{r=0..t} e^{d_r A} h0 + sum_{s<=t} C_t prod_{r=s+1..t} e^{d_r A} d_s B_s x_s ]
    + D x_t, written as explicit products (no recurrence)."""
    B, D, L = p["xh"].shape
    N = p["A"].shape[1]
    Gbc = p["Bh"].shape[1]
    y = np.zeros((B, D, L))
    for b, d, t in itertools.product(range(B), range(D), range(L)):
        g = d // (D // Gbc)
        tot = 0.0
        for n in range(N):
            a = p["A"][d, n]
            c = p["Ch"][b, g, n, t]
            if p["h0"] is not None:
                tot += c * math.prod(math.exp(p["delta"][b, d, r] * a) for r in range(t + 1)) * p["h0"][b, d, n]
            for s in range(t + 1):
                dec = math.prod(math.exp(p["delta"][b, d, r] * a) for r in range(s + 1, t + 1))
                tot += c * dec * p["delta"][b, d, s] * p["Bh"][b, g, n, s] * p["xh"][b, d, s]
        y[b, d, t] = tot + p["Dskip"][d] * p["xh"][b, d, t]
    return y


@pytest.mark.parametrize("Gbc,D", [(1, 3), (2, 4)])
def test_selective_scan_equals_unrolled_sum(Gbc, D):
    p = small_m1(seed=1, D=D, Gbc=Gbc)
    y, _ = oracle.selective_scan(**p)
    np.testing.assert_allclose(y, unrolled_y(p), rtol=1e-12, atol=1e-12)


def test_selective_scan_geometric_closed_form():
    B, D, L, N = 1, 2, 300, 3
    a_log, dt, bb, cc, xx = -0.7, 0.2, 1.3, -0.4, 2.5
    p = dict(xh=np.full((B, D, L), xx), delta=np.full((B, D, L), dt), A=np.full((D, N), a_log),
             Bh=np.full((B, 1, N, L), bb), Ch=np.full((B, 1, N, L), cc), Dskip=np.full(D, 0.3))
    y, hl = oracle.selective_scan(**p)
    a = math.exp(dt * a_log)
    b = dt * bb * xx
    t = np.arange(L)
    h = b * (1 - a ** (t + 1)) / (1 - a)
    np.testing.assert_allclose(y[0, 0], N * cc * h + 0.3 * xx, rtol=1e-12)
    np.testing.assert_allclose(hl[0, 1], h[-1], rtol=1e-12)


def test_selective_scan_zero_delta_keeps_state():
    p = small_m1(seed=2)
    p["delta"] = np.zeros_like(p["delta"])
    y, hl = oracle.selective_scan(**p)
    np.testing.assert_array_equal(hl, p["h0"])
    want = np.einsum("bgnl,bdn->bdl", p["Ch"], p["h0"]) + p["Dskip"][None, :, None] * p["xh"]
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-13)


def test_selective_scan_channel_permutation_commutes():
    """Quamba2 compute invariance: rearranging channels (x, delta, A, D, h0 alike) permutes y."""
    p = small_m1(seed=3, D=6)
    perm = np.array([4, 0, 5, 2, 1, 3])
    q = dict(p, xh=p["xh"][:, perm], delta=p["delta"][:, perm], A=p["A"][perm],
             Dskip=p["Dskip"][perm], h0=p["h0"][:, perm])
    y, hl = oracle.selective_scan(**p)
    yq, hq = oracle.selective_scan(**q)
    np.testing.assert_array_equal(yq, y[:, perm])
    np.testing.assert_array_equal(hq, hl[:, perm])


def test_selective_scan_split_resume():
    p = small_m1(seed=4, L=40)
    y, hl = oracle.selective_scan(**p)
    sl = lambda a, s: a[..., s]
    p1 = dict(p, xh=sl(p["xh"], slice(0, 17)), delta=sl(p["delta"], slice(0, 17)),
              Bh=sl(p["Bh"], slice(0, 17)), Ch=sl(p["Ch"], slice(0, 17)))
    y1, h1 = oracle.selective_scan(**p1)
    p2 = dict(p, xh=sl(p["xh"], slice(17, 40)), delta=sl(p["delta"], slice(17, 40)),
              Bh=sl(p["Bh"], slice(17, 40)), Ch=sl(p["Ch"], slice(17, 40)), h0=h1)
    y2, h2 = oracle.selective_scan(**p2)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=-1), y)
    np.testing.assert_array_equal(h2, hl)


def test_integer_codes_with_unit_scales_are_the_unquantized_scan():
    """All scales 1 and integer-valued x, B, C in [-128, 127]: quantize-dequantize is the identity,
    so the W8A8 path equals the scan of the raw values."""
    r = np.random.default_rng(5)
    B, D, L, N = 1, 4, 20, 4
    x = r.integers(-128, 128, (B, D, L)).astype(np.float32)
    Bm = r.integers(-128, 128, (B, 1, N, L)).astype(np.float32)
    qx = oracle.quant_group_x(x, np.zeros(D, np.uint8), np.ones(1, np.float32))
    qB = oracle.quant_state_group(Bm, 2, np.ones(2, np.float32))
    np.testing.assert_array_equal(oracle.dequant_group(qx, np.zeros(D, np.uint8), [1.0]), x)
    np.testing.assert_array_equal(oracle.dequant_state_group(qB, 2, [1.0, 1.0]), Bm)
    p = small_m1(seed=6, B=B, D=D, L=L, N=N)
    ya, _ = oracle.selective_scan(**dict(p, xh=oracle.dequant_group(qx, np.zeros(D, np.uint8), [1.0]),
                                         Bh=oracle.dequant_state_group(qB, 2, [1.0, 1.0])))
    yb, _ = oracle.selective_scan(**dict(p, xh=x.astype(np.float64), Bh=Bm.astype(np.float64)))
    np.testing.assert_array_equal(ya, yb)


def test_invalid_scale_groups_dequantize_to_zero():
    """A group whose scale is outside [2^-100, 2^100] (or NaN) holds codes 0 and values 0 (not
    0 * inf = NaN); the range ends themselves are valid."""
    q = np.full((1, 6, 3), 5, np.int8)
    scales = np.array([np.inf, np.nan, 2.0 ** 101, 1e-35, 2.0 ** -100, 2.0 ** 100], np.float32)
    v = oracle.dequant_group(q, np.arange(6, dtype=np.uint8), scales)
    np.testing.assert_array_equal(v[0, :4], 0.0)
    np.testing.assert_array_equal(v[0, 4], 5 * 2.0 ** -100)
    np.testing.assert_array_equal(v[0, 5], 5 * 2.0 ** 100)
    x = np.full((1, 6, 3), 3.0, np.float32)
    assert not oracle.quant_group_x(x, np.arange(6, dtype=np.uint8), scales)[0, :4].any()
    qb = np.full((1, 1, 4, 2), -7, np.int8)
    vb = oracle.dequant_state_group(qb, 2, np.array([np.inf, 0.5], np.float32))
    np.testing.assert_array_equal(vb[0, 0, :2], 0.0)
    np.testing.assert_array_equal(vb[0, 0, 2:], -3.5)


# ------------------------------------------------------------------------------------------------
# S4D

def test_zoh_matches_matrix_exponential():
    """Abar and Bbar from the exponential of the augmented real system [[ar, -ai, br], [ai, ar, bi],
    [0, 0, 0]] (state h = (re, im), input held constant over the step)."""
    r = np.random.default_rng(7)
    a = -np.exp(r.uniform(-2, 1, 16)) + 1j * r.uniform(-200, 200, 16)
    b = r.standard_normal(16) + 1j * r.standard_normal(16)
    for dt in (1e-3, 0.03, 0.1):
        Ab, Bb = oracle.s4d_zoh(a, b, dt)
        for k in range(16):
            M = np.array([[a[k].real, -a[k].imag, b[k].real], [a[k].imag, a[k].real, b[k].imag],
                          [0.0, 0.0, 0.0]])
            E = scipy.linalg.expm(M * dt)
            assert E[0, 0] == pytest.approx(Ab[k].real, rel=1e-9, abs=1e-12)
            assert E[1, 0] == pytest.approx(Ab[k].imag, rel=1e-9, abs=1e-12)
            assert E[0, 2] == pytest.approx(Bb[k].real, rel=1e-8, abs=1e-13)
            assert E[1, 2] == pytest.approx(Bb[k].imag, rel=1e-8, abs=1e-13)
        assert np.all(np.abs(Ab) < 1.0)


def test_zoh_zero_pole_limit():
    # Bbar = (e^{a dt} - 1)/a * b -> dt * b (1 + a dt / 2 + ...) as a -> 0
    a = np.array([0j, -1e-5 + 2e-5j])
    Ab, Bb = oracle.s4d_zoh(a, np.array([2 + 1j, 2 + 1j]), 0.05)
    assert Ab[0] == 1.0 and Bb[0] == 0.05 * (2 + 1j)
    want = 0.05 * (2 + 1j) * (1 + a[1] * 0.05 / 2)
    assert abs(Bb[1] - want) < 1e-10 * abs(want)


def s4d_small(seed=8, B=2, H=3, N=5, L=60):
    r = np.random.default_rng(seed)
    Ah = -np.exp(r.uniform(-1, 0.5, (H, N))) + 1j * np.pi * np.arange(N)[None, :]
    Bh = r.standard_normal((H, N)) + 1j * r.standard_normal((H, N))
    Ch = r.standard_normal((H, N)) + 1j * r.standard_normal((H, N))
    dt = np.exp(r.uniform(np.log(1e-3), np.log(1e-1), H))
    u = r.uniform(0, 1, (B, H, L))
    return u, Ah, Bh, Ch, dt, r.standard_normal(H)


def s4d_kernel(Ah, Bh, Ch, dt, L):
    H, N = Ah.shape
    K = np.zeros((H, L))
    for h in range(H):
        Ab, Bb = oracle.s4d_zoh(Ah[h], Bh[h], dt[h])
        powers = Ab[None, :] ** np.arange(L)[:, None]
        K[h] = np.real((Ch[h][None, :] * powers * Bb[None, :]).sum(axis=1))
    return K


def test_s4d_impulse_response_is_the_textbook_kernel():
    u, Ah, Bh, Ch, dt, D = s4d_small()
    L = u.shape[2]
    imp = np.zeros_like(u)
    imp[:, :, 0] = 1.0
    y, _ = oracle.s4d_scan(imp, Ah, Bh, Ch, dt, Dskip=D)
    K = s4d_kernel(Ah, Bh, Ch, dt, L)
    want = K[None] + D[None, :, None] * imp
    np.testing.assert_allclose(y, want, rtol=1e-10, atol=1e-12)


def test_s4d_recurrence_equals_convolution():
    u, Ah, Bh, Ch, dt, D = s4d_small(seed=9)
    B, H, L = u.shape
    y, _ = oracle.s4d_scan(u, Ah, Bh, Ch, dt, Dskip=D)
    K = s4d_kernel(Ah, Bh, Ch, dt, L)
    for b, h in itertools.product(range(B), range(H)):
        want = np.convolve(u[b, h], K[h])[:L] + D[h] * u[b, h]
        np.testing.assert_allclose(y[b, h], want, rtol=1e-9, atol=1e-11)


def test_s4d_split_resume_and_int16_state():
    u, Ah, Bh, Ch, dt, D = s4d_small(seed=10, L=50)
    y, hl = oracle.s4d_scan(u, Ah, Bh, Ch, dt, Dskip=D)
    y1, h1 = oracle.s4d_scan(u[..., :21], Ah, Bh, Ch, dt, Dskip=D)
    y2, h2 = oracle.s4d_scan(u[..., 21:], Ah, Bh, Ch, dt, Dskip=D, h0=h1)
    np.testing.assert_array_equal(np.concatenate([y1, y2], -1), y)
    np.testing.assert_array_equal(h2, hl)
    # int16 state: a pure-Python loop that rounds each part to the state grid after every step
    ss = np.full(Ah.shape[0], 1e-3)
    yq, hq = oracle.s4d_scan(u, Ah, Bh, Ch, dt, Dskip=D, state_scale=ss)
    B, H, L = u.shape
    for b, h in itertools.product(range(B), range(H)):
        Ab, Bb = oracle.s4d_zoh(Ah[h], Bh[h], dt[h])
        st = np.zeros(Ah.shape[1], dtype=np.complex128)
        for t in range(L):
            st = Ab * st + Bb * u[b, h, t]
            st = ss[h] * np.clip(np.rint(st.real / ss[h]), -32768, 32767) + \
                1j * ss[h] * np.clip(np.rint(st.imag / ss[h]), -32768, 32767)
            ref = np.real((Ch[h] * st).sum()) + D[h] * u[b, h, t]
            assert yq[b, h, t] == pytest.approx(ref, rel=1e-12, abs=1e-12)
        np.testing.assert_allclose(hq[b, h], st, rtol=0, atol=1e-15)
    assert np.all(np.abs(hq.real / 1e-3 - np.rint(hq.real / 1e-3)) < 1e-6)


# ------------------------------------------------------------------------------------------------
# SSD chunked form

def ssd_small(seed=11, B=2, L=40, nh=4, P=3, N=5, Gbc=2, h0=True):
    r = np.random.default_rng(seed)
    return dict(xh=r.standard_normal((B, L, nh, P)), delta=r.uniform(0.02, 0.6, (B, L, nh)),
                A=-np.exp(r.uniform(0, 2, nh)), Bh=r.standard_normal((B, L, Gbc, N)),
                Ch=r.standard_normal((B, L, Gbc, N)), Dskip=r.standard_normal(nh),
                h0=r.standard_normal((B, nh, P, N)) if h0 else None)


@pytest.mark.parametrize("Q", [1, 2, 7, 16, 40, 64])
def test_ssd_chunked_equals_sequential(Q):
    p = ssd_small()
    y, hl = oracle.ssd_chunked(chunk=Q, **p)
    ys, hs = oracle.ssd_as_sequential(**p)
    np.testing.assert_allclose(y, ys, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(hl, hs, rtol=1e-11, atol=1e-11)


def test_ssd_quadratic_attention_form_equals_sequential():
    """Duality: one chunk covering the sequence is the masked quadratic form
    Y = (L o C B^T) (delta x) with L_ij = exp(cum_i - cum_j) [j <= i] (plus the h0 and D terms),
    written here directly in numpy and compared with the sequential scan."""
    p = ssd_small(seed=12, L=25)
    B, L, nh, P = p["xh"].shape
    Gbc = p["Bh"].shape[2]
    ys, _ = oracle.ssd_as_sequential(**p)
    for b, h in itertools.product(range(B), range(nh)):
        g = h // (nh // Gbc)
        cum = np.cumsum(p["delta"][b, :, h] * p["A"][h])
        Lmask = np.tril(np.exp(cum[:, None] - cum[None, :]))
        CB = p["Ch"][b, :, g, :] @ p["Bh"][b, :, g, :].T
        Y = (Lmask * CB) @ (p["delta"][b, :, h][:, None] * p["xh"][b, :, h, :])
        Y += np.exp(cum)[:, None] * (p["Ch"][b, :, g, :] @ p["h0"][b, h].T)
        Y += p["Dskip"][h] * p["xh"][b, :, h, :]
        np.testing.assert_allclose(ys[b, :, h, :], Y, rtol=1e-10, atol=1e-10)


def test_ssd_int8_state_exact_in_its_special_case():
    """With A = 0 and a constant delta every weight w_j equals w_max, so the requantized operand is
    the x code itself and the int8 chunk state is exact."""
    r = np.random.default_rng(13)
    p = ssd_small(seed=13, L=50)
    B, L, nh, P = p["xh"].shape
    qx = r.integers(-128, 128, (B, L, nh, P)).astype(np.int8)
    sx = r.uniform(0.01, 0.1, nh * P)
    p.update(xh=qx * sx.reshape(nh, P), delta=np.full((B, L, nh), 0.37), A=np.zeros(nh))
    y0, h0_ = oracle.ssd_chunked(chunk=16, **p)
    y1, h1_ = oracle.ssd_chunked(chunk=16, int8_state=True, qx=qx, sx=sx, **p)
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h1_, h0_, rtol=1e-12, atol=1e-12)


def test_ssd_int8_state_error_is_small_generic():
    """Away from the special case the int8 chunk state approximates the exact one (not a pin:
    the requantization error of the method)."""
    r = np.random.default_rng(14)
    p = ssd_small(seed=14, L=64, P=8, N=8)
    B, L, nh, P = p["xh"].shape
    sx = np.full(nh * P, 3.0 / 127)
    qx = np.clip(np.rint(p["xh"] / 3.0 * 127), -128, 127).astype(np.int8)
    p["xh"] = qx * sx.reshape(nh, P)
    y0, _ = oracle.ssd_chunked(chunk=16, **p)
    y1, _ = oracle.ssd_chunked(chunk=16, int8_state=True, qx=qx, sx=sx, **p)
    assert np.abs(y1 - y0).max() < 0.05 * np.abs(y0).max()


@pytest.mark.parametrize("L,chunk", [(40, 64), (64, 16)])
def test_ssd_int8_state_within_its_requantization_bound(L, chunk):
    """Generic pin of the int8 chunk state. Since |qx| <= 128 and w_j <= w_max, qx*w_j/w_max lies
    in [-128, 127]: the saturation never acts and each requantized code r = RNE(qx*w_j/w_max) is
    within 1/2 of it, so per chunk
        |S_int8[p,n] - S_exact[p,n]| <= sx[p] * w_max / 2 * sum_j |B_j[n]|,
    and over chunks the state error is that chunk bound carried by the chunk decays. The bound is
    computed here from the method's definitions (cumsum, weights, decays) with h0 = 0, and the
    error must also reach a sizeable fraction of it (an exact or over-smoothed state would not)."""
    r = np.random.default_rng(17)
    p = ssd_small(seed=17, L=L, P=6, N=7, h0=False)
    B, _, nh, P = p["xh"].shape
    Gbc, N = p["Bh"].shape[2], p["Bh"].shape[3]
    sx = r.uniform(0.005, 0.05, nh * P)
    qx = r.integers(-128, 128, (B, L, nh, P)).astype(np.int8)
    p["xh"] = qx * sx.reshape(nh, P)
    _, h_exact = oracle.ssd_chunked(chunk=chunk, **p)
    _, h_int8 = oracle.ssd_chunked(chunk=chunk, int8_state=True, qx=qx, sx=sx, **p)
    hpg = nh // Gbc
    worst = 0.0
    for b, h in itertools.product(range(B), range(nh)):
        g = h // hpg
        bound = np.zeros((P, N))
        for t0 in range(0, L, chunk):
            dt = p["delta"][b, t0:t0 + chunk, h]
            cum = np.cumsum(dt * p["A"][h])
            w = dt * np.exp(cum[-1] - cum)
            absB = np.abs(p["Bh"][b, t0:t0 + chunk, g, :]).sum(axis=0)
            chunk_bound = sx[h * P:(h + 1) * P, None] * (w.max() / 2) * absB[None, :]
            bound = np.exp(cum[-1]) * bound + chunk_bound
        err = np.abs(h_int8[b, h] - h_exact[b, h])
        assert np.all(err <= bound * (1 + 1e-9) + 1e-15), (b, h)
        worst = max(worst, (err / bound).max())
    assert worst > 0.05


def test_ssd_int8_state_rounding_is_unbiased():
    """Round-to-nearest-even of the requantized codes has no bias: with B >= 0 and x codes >= 0
    every rounding error enters the chunk state with the same sign of weight, so a floor, ceiling
    or truncation would move
    the state by about the whole bound of the test above in one direction, while RNE errors
    average out (the mean signed error stays a small fraction of the mean bound)."""
    r = np.random.default_rng(18)
    p = ssd_small(seed=18, L=64, P=6, N=7, h0=False)
    B, L, nh, P = p["xh"].shape
    p["Bh"] = np.abs(p["Bh"])
    # weak decay and delta in [0.3, 0.6]: every w_j / w_max lies in about [0.5, 1], so the
    # fractional parts of the scaled codes spread evenly (small weights would all round to 0,
    # a one-sided error of the method itself, not of its rounding rule)
    p["A"] = np.full(nh, -0.01)
    p["delta"] = r.uniform(0.3, 0.6, (B, L, nh))
    sx = r.uniform(0.005, 0.05, nh * P)
    qx = r.integers(0, 128, (B, L, nh, P)).astype(np.int8)  # one sign: truncation is biased too
    p["xh"] = qx * sx.reshape(nh, P)
    _, h_exact = oracle.ssd_chunked(chunk=L, **p)
    _, h_int8 = oracle.ssd_chunked(chunk=L, int8_state=True, qx=qx, sx=sx, **p)
    Gbc = p["Bh"].shape[2]
    signed, bounds = [], []
    for b, h in itertools.product(range(B), range(nh)):
        dt = p["delta"][b, :, h]
        cum = np.cumsum(dt * p["A"][h])
        w = dt * np.exp(cum[-1] - cum)
        absB = p["Bh"][b, :, h // (nh // Gbc), :].sum(axis=0)
        bounds.append(sx[h * P:(h + 1) * P, None] * (w.max() / 2) * absB[None, :])
        signed.append(h_int8[b, h] - h_exact[b, h])
    ratio = np.mean(signed) / np.mean(bounds)
    assert abs(ratio) < 0.2, ratio


# ------------------------------------------------------------------------------------------------
# Decode

def test_decode_steps_equal_sequential_scan():
    r = np.random.default_rng(15)
    B, nh, P, N, Gbc, K = 2, 4, 3, 5, 2, 6
    xs = r.standard_normal((K, B, nh, P))
    Bs = r.standard_normal((K, B, Gbc, N))
    Cs = r.standard_normal((K, B, Gbc, N))
    ds = r.uniform(0.05, 0.5, (K, B, nh))
    A = -np.exp(r.uniform(0, 2, nh))
    D = r.standard_normal(nh)
    st0 = r.standard_normal((B, nh, P, N))
    st = st0.copy()
    ys = [oracle.decode_step(xs[k], Bs[k], Cs[k], ds[k], A, st, Dskip=D) for k in range(K)]
    # the same K tokens as one length-K sequence through the SSD sequential scan
    yseq, hseq = oracle.ssd_as_sequential(xs.transpose(1, 0, 2, 3), ds.transpose(1, 0, 2), A,
                                          Bs.transpose(1, 0, 2, 3), Cs.transpose(1, 0, 2, 3),
                                          Dskip=D, h0=st0)
    np.testing.assert_allclose(np.stack(ys, 1), yseq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, hseq, rtol=1e-12, atol=1e-12)


def test_decode_zero_delta():
    r = np.random.default_rng(16)
    B, nh, P, N, Gbc = 1, 2, 3, 4, 1
    st = r.standard_normal((B, nh, P, N))
    st0 = st.copy()
    x, Bm, Cm = r.standard_normal((B, nh, P)), r.standard_normal((B, Gbc, N)), r.standard_normal((B, Gbc, N))
    D = r.standard_normal(nh)
    y = oracle.decode_step(x, Bm, Cm, np.zeros((B, nh)), -np.ones(nh), st, Dskip=D)
    np.testing.assert_array_equal(st, st0)
    np.testing.assert_allclose(y, np.einsum("bhpn,bn->bhp", st0, Cm[:, 0]) + D[None, :, None] * x,
                               rtol=1e-13)


# ------------------------------------------------------------------------------------------------
# the per-row error measure used by every parity test

def test_rowwise_error_measure():
    # max |y - r| over the row divided by max |r| of the row
    assert np.allclose(oracle.rowwise_error([[1.0, 2.0], [3.0, 5.0]], [[1.0, 4.0], [3.0, 4.0]]),
                       [0.5, 0.25])
    # complex rows (the S4D state) are measured by the modulus: an error in the imaginary part
    # alone counts in full
    assert np.allclose(oracle.rowwise_error([[1.0 + 1.0j, 0.0]], [[1.0 + 0.0j, 0.0]]), [1.0])
    assert np.allclose(oracle.rowwise_error([[3.0 + 4.0j]], [[0.0 + 0.0j]], axis=-1) > 1e6, [True])
    # an all-zero reference row is floored at 1e-6 of the largest reference value
    assert np.allclose(oracle.rowwise_error([[1e-3], [2.0]], [[0.0], [2.0]]), [500.0, 0.0])


# ------------------------------------------------------------------------------------------------
# int16 S4D state: worked closed forms (A = 0, so Abar = 1 and Bbar = dt * B exactly) and a
# deterministic rounding-error bound against the unrounded fp64 run

def s4d_const_increment(inc_re, inc_im, s, L, C=1.0 + 0.5j, D=0.25):
    """One channel, one state, A = 0, dt = 1, B = (inc_re + i inc_im) * s, u = 1 at every step."""
    u = np.ones((1, 1, L))
    Ah = np.zeros((1, 1), np.complex128)
    Bh = np.full((1, 1), (inc_re + 1j * inc_im) * s)
    Ch = np.full((1, 1), C)
    return oracle.s4d_scan(u, Ah, Bh, Ch, np.ones(1), Dskip=np.full(1, D),
                           state_scale=np.full(1, s))


def test_s4d_int16_dead_zone():
    """Increments of 0.3 grid steps round back to 0 after every step: the int16 state never leaves
    0, y is the D term alone. (Rounding before adding the input would hold 0.3 s; rounding only at
    the readout would let the state grow as 0.3 t s.)"""
    s = 2.0 ** -10
    y, hl = s4d_const_increment(0.3, -0.3, s, 40)
    assert np.all(hl == 0)
    assert np.all(y == 0.25)


def test_s4d_int16_exact_walk_and_saturation():
    """Increments of 0.6 grid steps (real part): h_t = round(h_{t-1} + 0.6) = t exactly. Increments
    of -1000.25 grid steps (imaginary part): -1000 t until the code saturates at -32768 (t = 33),
    where it stays. Every y_t is Re(C h_t) + D with those exact states."""
    s = 2.0 ** -12
    L = 50
    C, D = 1.0 + 0.5j, 0.25
    y, hl = s4d_const_increment(0.6, -1000.25, s, L, C=C, D=D)
    t = np.arange(1, L + 1)
    h = t * s + 1j * np.maximum(-1000.0 * t, -32768.0) * s
    np.testing.assert_array_equal(hl[0, 0, 0], h[-1])
    np.testing.assert_array_equal(y[0, 0], (C * h).real + D)
    # positive saturation at +32767
    y2, hl2 = s4d_const_increment(1000.25, 0.0, s, L, C=C, D=D)
    h2 = np.minimum(1000.0 * t, 32767.0) * s
    np.testing.assert_array_equal(hl2[0, 0, 0], h2[-1] + 0j)
    np.testing.assert_array_equal(y2[0, 0], C.real * h2 + D)


def test_s4d_int16_error_bound_against_fp64():
    """Generic channels: per step each part is rounded by at most s/2, so the state error obeys
    e_t = Abar e_{t-1} + r_t with |r_t| <= s / sqrt(2), hence |e_t| <= s / sqrt(2) * sum_{k<t}
    |Abar|^k, and |y_t - y_t(fp64)| <= sum_n |C_n| |e_t,n|. Checked at every step (states below
    the saturation limit); the int16 run must also sit on the grid and differ from the fp64 run."""
    u, Ah, Bh, Ch, dt, D = s4d_small(seed=12, L=60)
    B, H, L = u.shape
    s = np.full(H, 2.0 ** -9)
    yq, hq = oracle.s4d_scan(u, Ah, Bh, Ch, dt, Dskip=D, state_scale=s)
    y, hl = oracle.s4d_scan(u, Ah, Bh, Ch, dt, Dskip=D)
    for h in range(H):
        Ab, _ = oracle.s4d_zoh(Ah[h], Bh[h], dt[h])
        geo = np.cumsum(np.abs(Ab)[None, :] ** np.arange(L)[:, None], axis=0)   # [t, n]
        ebound = s[h] / np.sqrt(2.0) * geo
        ybound = (np.abs(Ch[h])[None, :] * ebound).sum(axis=1)
        for b in range(B):
            assert np.all(np.abs(yq[b, h] - y[b, h]) <= ybound * (1 + 1e-9) + 1e-12)
            assert np.all(np.abs(hq[b, h] - hl[b, h]) <= ebound[-1] * (1 + 1e-9) + 1e-12)
            assert np.all(np.abs(hl[b, h].real) < 30000 * s[h])
    grid = np.concatenate([hq.real.ravel(), hq.imag.ravel()]) / s[0]
    assert np.array_equal(grid, np.rint(grid))
    assert not np.array_equal(hq, hl)


# ------------------------------------------------------------------------------------------------
# int8 intra-chunk output (row-requantized intra-chunk weights times the x codes)

def intra_weights(p, b, h, t0, q, hpg):
    """W[i, j] = (C_i . B_j) exp(cum_i - cum_j) delta_j [j <= i] of one chunk, from the method's
    definitions written out in numpy."""
    g = h // hpg
    dt = p["delta"][b, t0:t0 + q, h]
    cum = np.cumsum(dt * p["A"][h])
    CB = p["Ch"][b, t0:t0 + q, g, :] @ p["Bh"][b, t0:t0 + q, g, :].T
    return np.tril(CB * np.exp(cum[:, None] - cum[None, :]) * dt[None, :])


def test_ssd_int8_intra_exact_in_its_special_case():
    """A = 0 and delta = 1 make W = C B^T; with one-hot C (state 0) and B[:, 0] integral with
    B[0, 0] = 127, every row's largest |W| is 127, so each requantized weight equals W itself and
    the int8 intra-chunk output is exact (the state, x codes and D term unchanged)."""
    r = np.random.default_rng(31)
    p = ssd_small(seed=31, L=48)
    B, L, nh, P = p["xh"].shape
    Gbc, N = p["Bh"].shape[2], p["Bh"].shape[3]
    qx = r.integers(-128, 128, (B, L, nh, P)).astype(np.int8)
    sx = r.uniform(0.01, 0.1, nh * P)
    Ch = np.zeros((B, L, Gbc, N))
    Ch[..., 0] = 1.0
    Bh = np.zeros((B, L, Gbc, N))
    Bh[..., 0] = r.integers(-127, 128, (B, L, Gbc))
    Bh[:, ::16, :, 0] = 127.0  # the first step of every 16-step chunk
    p.update(xh=qx * sx.reshape(nh, P), delta=np.ones((B, L, nh)), A=np.zeros(nh), Ch=Ch, Bh=Bh)
    y0, h0_ = oracle.ssd_chunked(chunk=16, **p)
    y1, h1_ = oracle.ssd_chunked(chunk=16, int8_intra=True, qx=qx, sx=sx, **p)
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(h1_, h0_)


@pytest.mark.parametrize("L,chunk", [(40, 64), (64, 16), (50, 7)])
def test_ssd_int8_intra_within_its_requantization_bound(L, chunk):
    """Generic pin. Each requantized weight is within half a step m_i / 254 of W[i, j] (|W| <=
    m_i keeps it inside +-127), so per output
        |y_int8[i, p] - y_exact[i, p]| <= (m_i / 254) * sum_{j <= i} |xh_j[p]|,
    with m_i the row's largest |W| computed here from the definitions; the state is untouched.
    The error must also reach a sizeable fraction of the bound (an exact or smoothed output
    would not)."""
    r = np.random.default_rng(32)
    p = ssd_small(seed=32, L=L, P=6, N=7, h0=True)
    B, _, nh, P = p["xh"].shape
    Gbc = p["Bh"].shape[2]
    sx = r.uniform(0.005, 0.05, nh * P)
    qx = r.integers(-128, 128, (B, L, nh, P)).astype(np.int8)
    p["xh"] = qx * sx.reshape(nh, P)
    y_exact, h_exact = oracle.ssd_chunked(chunk=chunk, **p)
    y_int8, h_int8 = oracle.ssd_chunked(chunk=chunk, int8_intra=True, qx=qx, sx=sx, **p)
    np.testing.assert_array_equal(h_int8, h_exact)
    hpg = nh // Gbc
    worst = 0.0
    for b, h in itertools.product(range(B), range(nh)):
        for t0 in range(0, L, chunk):
            q = min(chunk, L - t0)
            W = intra_weights(p, b, h, t0, q, hpg)
            m = np.abs(W).max(axis=1)
            ax = np.abs(p["xh"][b, t0:t0 + q, h, :])
            bound = (m / 254)[:, None] * np.cumsum(ax, axis=0)
            err = np.abs(y_int8[b, t0:t0 + q, h, :] - y_exact[b, t0:t0 + q, h, :])
            assert np.all(err <= bound * (1 + 1e-9) + 1e-13), (b, h, t0)
            worst = max(worst, (err / np.maximum(bound, 1e-300)).max())
    assert worst > 0.05


def test_ssd_int8_intra_rounding_is_unbiased():
    """With W >= 0 (C, B >= 0) and x codes >= 0 every rounding error of the requantized weights
    enters with the same sign of weight: a floor, ceiling or truncation would shift the outputs by
    a large part of the bound above in one direction, while round-to-nearest-even errors average
    out."""
    r = np.random.default_rng(33)
    p = ssd_small(seed=33, L=64, P=6, N=7, h0=False)
    B, L, nh, P = p["xh"].shape
    Gbc = p["Bh"].shape[2]
    p["Bh"] = np.abs(p["Bh"])
    p["Ch"] = np.abs(p["Ch"])
    p["A"] = np.full(nh, -0.01)
    p["delta"] = r.uniform(0.3, 0.6, (B, L, nh))
    sx = r.uniform(0.005, 0.05, nh * P)
    qx = r.integers(0, 128, (B, L, nh, P)).astype(np.int8)
    p["xh"] = qx * sx.reshape(nh, P)
    y_exact, _ = oracle.ssd_chunked(chunk=L, **p)
    y_int8, _ = oracle.ssd_chunked(chunk=L, int8_intra=True, qx=qx, sx=sx, **p)
    signed, bounds = [], []
    for b, h in itertools.product(range(B), range(nh)):
        W = intra_weights(p, b, h, 0, L, nh // Gbc)
        m = np.abs(W).max(axis=1)
        bounds.append((m / 254)[:, None] * np.cumsum(np.abs(p["xh"][b, :, h, :]), axis=0))
        signed.append(y_int8[b, :, h, :] - y_exact[b, :, h, :])
    ratio = np.mean(signed) / np.mean(bounds)
    assert abs(ratio) < 0.2, ratio


def test_ssd_int8_intra_and_state_modes_compose():
    """Both int8 modes at once: the intra-chunk output of the combined run equals that of the
    intra-only run where the state does not enter (first chunk, no h0), and its state equals the
    state-only run's."""
    r = np.random.default_rng(34)
    p = ssd_small(seed=34, L=40, P=6, N=7, h0=False)
    B, L, nh, P = p["xh"].shape
    sx = r.uniform(0.005, 0.05, nh * P)
    qx = r.integers(-128, 128, (B, L, nh, P)).astype(np.int8)
    p["xh"] = qx * sx.reshape(nh, P)
    y_i, _ = oracle.ssd_chunked(chunk=16, int8_intra=True, qx=qx, sx=sx, **p)
    _, h_s = oracle.ssd_chunked(chunk=16, int8_state=True, qx=qx, sx=sx, **p)
    y_b, h_b = oracle.ssd_chunked(chunk=16, int8_intra=True, int8_state=True, qx=qx, sx=sx, **p)
    np.testing.assert_array_equal(y_b[:, :16], y_i[:, :16])
    np.testing.assert_array_equal(h_b, h_s)
