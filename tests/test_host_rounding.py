"""The library's rounding helpers (quantized_state_space_amd/csrc/common.hpp), built for the host,
against the oracle's exact quantizer and soft-edge encoder: every fp32 value of whole binades around
the saturation edge and near zero, constructed ties and their neighbours, special values and
scales at the ends of the valid range. CPU only; the GPU tests check the same helpers as compiled
for gfx950 inside the kernels."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import qssm_synth as synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def hr(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("hr") / "libhr.so")
    subprocess.check_call([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-ffp-contract=off",
                           "-fPIC", "-shared", "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "host_rounding.cpp"), "-o", out])
    lib = ctypes.CDLL(out)
    P, I64, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    lib.host_quant8.argtypes = [P, I64, F, P]
    lib.host_quant8_div.argtypes = [P, I64, F, P]
    lib.host_softedge.argtypes = [P, I64, F, F, F, ctypes.c_int32, P]
    return lib


def binade(e, sign=1.0):
    """All fp32 values with biased exponent e (and the given sign)."""
    bits = (np.uint32(e) << np.uint32(23)) | np.arange(1 << 23, dtype=np.uint32)
    v = bits.view(np.float32)
    return v if sign > 0 else -v


def host_codes(hr, fn, v, *args):
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8 if fn == "host_softedge" else np.int8)
    args = [int(a) if isinstance(a, int) else float(a) for a in args]
    getattr(hr, fn)(v.ctypes.data, v.size, *args, out.ctypes.data)
    return out


def oracle_codes(v, s):
    v = np.ascontiguousarray(v, dtype=np.float32)
    return oracle.quant_group_x(v.reshape(1, 1, -1), np.zeros(1, np.uint8),
                                np.float32([s])).reshape(-1)


def oracle_softedge(v, s, L, H, ratio=4):
    v = np.ascontiguousarray(v, dtype=np.float32)
    return oracle.softedge_encode(v.reshape(1, 1, -1), np.zeros(1, np.uint8), np.float32([s]),
                                  np.float32([L]), np.float32([H]), ratio=ratio).reshape(-1)


def ties_and_neighbours(s, rng, n=200000):
    k = rng.integers(-300, 300, n)
    v = ((k + 0.5) * np.float64(s)).astype(np.float32)
    up = np.nextafter(v, np.float32(np.inf))
    dn = np.nextafter(v, np.float32(-np.inf))
    return np.concatenate([v, up, dn, (k * np.float64(s)).astype(np.float32)])


def exponent_of(x):
    return int((np.float32(x).view(np.uint32) >> np.uint32(23)) & np.uint32(0xFF))


@pytest.mark.parametrize("s", [np.float32(0.0371), np.float32(3.0) / np.float32(7.0)])
def test_quant_whole_binades(hr, s):
    # |v/s| in [64, 256): the saturation edge; and values just above the first rounding boundary
    e = exponent_of(np.float32(64.0) * s)
    vals = [binade(e), binade(e, -1.0), binade(e + 1), binade(e + 1, -1.0),
            binade(exponent_of(np.float32(0.5) * s)), binade(exponent_of(np.float32(0.5) * s), -1.0)]
    for v in vals:
        got = host_codes(hr, "host_quant8", v, s)
        want = oracle_codes(v, s)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("s", [np.float32(2.0 ** -100), np.float32(2.0 ** 100),
                               np.float32(1e-30), np.float32(12345.678), np.float32(1.0),
                               np.float32(0.1), np.float32(7.0) / np.float32(3.0)])
def test_quant_ties_neighbours_and_edges(hr, s):
    rng = np.random.default_rng(int(np.float32(s).view(np.uint32)))
    v = np.concatenate([ties_and_neighbours(s, rng), synth.quantizer_edge_values(scale=s, n=20000)])
    got = host_codes(hr, "host_quant8", v, s)
    want = oracle_codes(v, s)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:5]]
    # the division form gives the same codes
    assert np.array_equal(host_codes(hr, "host_quant8_div", v, s), want)


@pytest.mark.parametrize("s", [np.float32(np.nan), np.float32(0.0), np.float32(-1.0),
                               np.float32(np.inf), np.float32(2.0 ** -101), np.float32(2.0 ** 101)])
def test_quant_invalid_scales_give_zero(hr, s):
    v = np.float32([0.0, 1.0, -1.0, 1e30, -1e30, np.inf, -np.inf, np.nan, 1e-40])
    assert not host_codes(hr, "host_quant8", v, s).any()


@pytest.mark.parametrize("ratio", [4, 2])
@pytest.mark.parametrize("s,L,H", [(np.float32(0.05), np.float32(0.1), np.float32(3.15)),
                                   (np.float32(1.0), np.float32(0.0), np.float32(63.0)),
                                   (np.float32(0.02), np.float32(0.5), np.float32(0.25)),
                                   (np.float32(2.0 ** -100), np.float32(1e-30), np.float32(3e-29))])
def test_softedge_matches_oracle(hr, s, L, H, ratio):
    rng = np.random.default_rng(5)
    parts = [ties_and_neighbours(s, rng, 50000),
             ties_and_neighbours(np.float32(s / ratio), rng, 50000),
             ties_and_neighbours(np.float32(s * ratio), rng, 50000),
             synth.quantizer_edge_values(scale=s, n=20000),
             np.float32([L, -L, H, -H, np.nextafter(L, 0), np.nextafter(H, np.inf), 0.0, -0.0,
                         np.inf, -np.inf, np.nan])]
    e = exponent_of(np.float32(16.0) * s)
    parts += [binade(e), binade(e, -1.0), binade(exponent_of(np.float32(4.0) * H))]
    v = np.concatenate(parts).astype(np.float32)
    got = host_codes(hr, "host_softedge", v, s, L, H, ratio)
    want = oracle_softedge(v, s, L, H, ratio)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]
