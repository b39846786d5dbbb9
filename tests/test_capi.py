"""C-ABI checks that need no GPU: the library loads, exports every function include/qssm.h
declares, reports argument errors before any launch, and its host calibration helpers agree with the
oracle bit for bit."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import qssm_synth as synth
import quantized_state_space_amd as qs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qssm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qssm_[a-z0-9_A-Z]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 18
    out = subprocess.run(["nm", "-D", "--defined-only", qs.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (qssm_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = qs.load()
    for n in names:
        assert hasattr(lib, n)
    assert set(qs.SIGNATURES) == set(names)


def test_struct_layouts_and_version():
    lib = qs.load()
    for kind, st in qs.ARG_STRUCTS.items():
        assert lib.qssm_args_size(kind) == ctypes.sizeof(st)
    assert lib.qssm_args_size(99) == 0
    assert lib.qssm_version() == 110
    assert lib.qssm_status_string(qs.QSSM_ERR_WORKSPACE) == b"workspace missing or too small"


def status(name, *args):
    lib = qs.load()
    return getattr(lib, name)(*args), lib.qssm_last_error().decode()


def test_quantizer_argument_errors_return_before_launch():
    dummy = ctypes.c_void_p(16)
    s, msg = status("qssm_quant_group_x", dummy, 1, 4, 4, None, dummy, 0, dummy, 0, dummy, None)
    assert s == qs.QSSM_ERR_INVALID_ARG and "G must be" in msg
    s, msg = status("qssm_quant_group_x", dummy, 1, 4, 4, None, dummy, 257, dummy, 0, dummy, None)
    assert s == qs.QSSM_ERR_INVALID_ARG
    s, msg = status("qssm_quant_group_x", None, 1, 4, 4, None, dummy, 1, dummy, 0, dummy, None)
    assert s == qs.QSSM_ERR_INVALID_ARG and "null" in msg
    s, msg = status("qssm_quant_group_x", dummy, -1, 4, 4, None, dummy, 1, dummy, 0, dummy, None)
    assert s == qs.QSSM_ERR_INVALID_ARG and "negative" in msg
    s, msg = status("qssm_quant_state_group_BC", dummy, 1, 2, 16, 4, 5, dummy, 0, dummy, None)
    assert s == qs.QSSM_ERR_INVALID_ARG and "divide" in msg
    s, msg = status("qssm_softedge_encode", dummy, 1, 4, 4, None, dummy, 1, None, dummy, dummy,
                    dummy, None)
    assert s == qs.QSSM_ERR_INVALID_ARG


def test_scan_argument_errors():
    lib = qs.load()
    a = qs.ScanArgs(batch=1, seqlen=8, dim=64, dstate=16, x_code=5, x_groups=1, bc_groups=1,
                    bc_group_size=4, y_dtype=0)
    assert lib.qssm_scan_w8a8(ctypes.byref(a), None, 0, None) == qs.QSSM_ERR_INVALID_ARG
    a.x_code = 0
    a.dstate = 12
    assert lib.qssm_scan_w8a8(ctypes.byref(a), None, 0, None) == qs.QSSM_ERR_UNSUPPORTED
    a.dstate = 16
    a.bc_group_size = 5
    assert lib.qssm_scan_w8a8(ctypes.byref(a), None, 0, None) == qs.QSSM_ERR_INVALID_ARG
    a.bc_group_size = 4
    assert lib.qssm_scan_w8a8(ctypes.byref(a), None, 0, None) == qs.QSSM_ERR_INVALID_ARG  # nulls
    assert b"null" in lib.qssm_last_error()
    p = ctypes.c_void_p(256)
    for f in ("x", "x_group_of", "x_scales", "delta", "A", "Bq", "Cq", "B_scales", "C_scales", "y"):
        setattr(a, f, p)
    need = lib.qssm_scan_workspace_size(ctypes.byref(a))
    assert need >= 1 * 1 * 16 * 8 * 2 * 4
    assert lib.qssm_scan_w8a8(ctypes.byref(a), p, need - 300, None) == qs.QSSM_ERR_WORKSPACE
    assert lib.qssm_scan_w8a8(None, None, 0, None) == qs.QSSM_ERR_INVALID_ARG


def test_other_entry_point_argument_errors():
    lib = qs.load()
    s4 = qs.S4dArgs(batch=1, seqlen=4, channels=2, dstate=4, state_dtype=qs.QSSM_I16)
    assert lib.qssm_s4d_scan(ctypes.byref(s4), None) == qs.QSSM_ERR_INVALID_ARG  # no state_scale
    s4.state_dtype = 7
    assert lib.qssm_s4d_scan(ctypes.byref(s4), None) == qs.QSSM_ERR_INVALID_ARG
    u = qs.UpdateArgs(batch=1, nheads=4, headdim=8, dstate=12, ngroups=3, x_groups=1,
                      bc_group_size=4, state_dtype=0)
    assert lib.qssm_state_update(ctypes.byref(u), None) == qs.QSSM_ERR_INVALID_ARG  # ngroups
    u.ngroups = 2
    assert lib.qssm_state_update(ctypes.byref(u), None) == qs.QSSM_ERR_UNSUPPORTED  # dstate 12
    u.dstate, u.bc_group_size, u.state_dtype = 4, 4, qs.QSSM_F16
    assert lib.qssm_state_update(ctypes.byref(u), None) == qs.QSSM_ERR_UNSUPPORTED  # fp16, N < 8
    sd = qs.SsdArgs(batch=1, seqlen=8, nheads=2, headdim=64, dstate=128, ngroups=1, chunk=256,
                    x_groups=1, bc_group_size=16, y_dtype=0)
    assert lib.qssm_ssd_chunk_int8(ctypes.byref(sd), None, 0, None) != qs.QSSM_OK
    # y offsets are 32-bit in the output kernel: more than 2^14 heads is refused before launch
    sd.nheads, sd.ngroups = (1 << 14) + 2, 2
    assert lib.qssm_ssd_chunk_int8(ctypes.byref(sd), None, 0, None) == qs.QSSM_ERR_UNSUPPORTED
    assert b"nheads" in lib.qssm_last_error()
    # the workspace size covers the fp16 chunk states, their factors and the staged tables
    sd.nheads, sd.ngroups, sd.seqlen, sd.batch = 4, 1, 600, 2
    nc, nh = 3, 4
    assert lib.qssm_ssd_workspace_size(ctypes.byref(sd)) >= (
        2 * nc * nh * 64 * 128 * 2 * 2 + 2 * nc * nh * 4 * 2 + nh * 64 * 4 + 2 * nc * nh * 256 * 4)


# ------------------------------------------------------------------------------------------------
# host calibration == oracle calibration, bit for bit

def test_channel_absmax_and_scales_match_oracle():
    inp = synth.c3_inputs(batch=1, seqlen=256, dim=96, calib_batch=1)
    x = inp["x_cal"].copy()
    x[0, 3, 5] = np.nan
    x[0, 7, 9] = np.inf
    got = qs.qssm_calib_channel_absmax(x)
    want = oracle.finite_absmax(x, axis=(0, 2))
    assert np.array_equal(got, want)
    a = np.concatenate([got, np.array([0.0, 1e-35, 3e38], np.float32)])
    assert np.array_equal(qs.qssm_calib_scales(a), oracle.scale_from_absmax(a))
    with pytest.raises(qs.QssmError):
        qs.qssm_calib_scales(np.array([np.nan], np.float32))


def test_channel_error_mean_matches_oracle():
    """Both accumulate the differences in fp64 (in different orders) and round the mean to fp32:
    equal to within one fp32 rounding of the mean."""
    r = np.random.default_rng(8)
    ref = r.standard_normal((3, 40, 257)).astype(np.float32)
    approx = (ref + 0.01 * r.standard_normal(ref.shape) + np.linspace(-0.1, 0.1, 40)[None, :, None]
              ).astype(np.float32)
    got = qs.qssm_calib_channel_error_mean(ref, approx)
    want = oracle.channel_error_mean(ref, approx)
    assert got.dtype == np.float32
    assert np.all(np.abs(got - want) <= np.spacing(np.abs(want).astype(np.float32)))
    bad = ref.copy()
    bad[1, 2, 3] = np.inf
    with pytest.raises(qs.QssmError, match="not finite"):
        qs.qssm_calib_channel_error_mean(bad, approx)


@pytest.mark.parametrize("C,G,seed", [(12, 4, 0), (64, 1, 1), (96, 8, 2), (1536, 8, 3), (300, 7, 4)])
def test_cluster_matches_oracle(C, G, seed):
    r = np.random.default_rng(seed)
    absmax = np.abs(r.standard_t(3, C) * np.where(r.random(C) < 0.01, 100, 1)).astype(np.float32)
    absmax[::17] = absmax[0]  # ties
    p1, g1 = qs.qssm_calib_cluster_channels(absmax, G)
    p2, g2 = oracle.cluster_channels(absmax, G)
    assert np.array_equal(p1, p2) and np.array_equal(g1, g2)


def test_softedge_thresholds_match_oracle():
    r = np.random.default_rng(9)
    v1 = r.standard_t(3, 100001).astype(np.float32)
    v2 = (r.standard_normal(77777) * 2).astype(np.float32)
    s, L, H, st = qs.qssm_calib_softedge(v1)
    os_, oL, oH, ost = oracle.softedge_thresholds(v1)
    assert (s, L, H) == (os_, oL, oH)
    s2, L2, H2, _ = qs.qssm_calib_softedge(v2, ema_state=st)
    os2, oL2, oH2, _ = oracle.softedge_thresholds(v2, prev=ost)
    assert (s2, L2, H2) == (os2, oL2, oH2)
