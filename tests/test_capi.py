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
    assert lib.qssm_version() == 180
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
                    qs.QSSM_X_SOFTEDGE, dummy, None)
    assert s == qs.QSSM_ERR_INVALID_ARG
    s, msg = status("qssm_softedge_encode", dummy, 1, 4, 4, None, dummy, 1, dummy, dummy, dummy,
                    qs.QSSM_X_INT8, dummy, None)
    assert s == qs.QSSM_ERR_INVALID_ARG and "form" in msg
    s, msg = status("qssm_softedge_decode", dummy, 1, 4, 4, dummy, 1, dummy, 7, dummy, None)
    assert s == qs.QSSM_ERR_INVALID_ARG and "form" in msg


def test_softedge_track_argument_errors():
    lib = qs.load()
    assert lib.qssm_softedge_track_workspace_size(0) == 0
    assert lib.qssm_softedge_track_workspace_size(33) == 0
    need = lib.qssm_softedge_track_workspace_size(8)
    assert need >= 8 * 4 * 256 * 8
    dummy = ctypes.c_void_p(256)
    s, msg = status("qssm_softedge_track", dummy, 1, 4, 4, None, dummy, 33, 0.1, 0, dummy, dummy,
                    dummy, dummy, dummy, 1 << 20, None)
    assert s == qs.QSSM_ERR_INVALID_ARG and "G must be" in msg
    s, msg = status("qssm_softedge_track", dummy, 1, 4, 4, None, dummy, 2, 1.5, 0, dummy, dummy,
                    dummy, dummy, dummy, 1 << 20, None)
    assert s == qs.QSSM_ERR_INVALID_ARG and "alpha" in msg
    s, msg = status("qssm_softedge_track", dummy, 1, 4, 4, None, dummy, 8, 0.1, 0, dummy, dummy,
                    dummy, dummy, dummy, need - 1, None)
    assert s == qs.QSSM_ERR_WORKSPACE
    s, msg = status("qssm_softedge_track", dummy, 1, 4, 4, None, dummy, 8, 0.1, 0, None, dummy,
                    dummy, dummy, dummy, need, None)
    assert s == qs.QSSM_ERR_INVALID_ARG and "null" in msg


def test_scan_argument_errors():
    lib = qs.load()
    a = qs.ScanArgs(batch=1, seqlen=8, dim=64, dstate=16, x_code=5, x_groups=1, bc_groups=1,
                    bc_group_size=4, y_dtype=0)
    assert lib.qssm_scan_w8a8(ctypes.byref(a), None, 0, None) == qs.QSSM_ERR_INVALID_ARG
    a.x_code = 0
    a.bc_code = 3
    assert lib.qssm_scan_w8a8(ctypes.byref(a), None, 0, None) == qs.QSSM_ERR_INVALID_ARG
    assert "bc_code" in lib.qssm_last_error().decode()
    a.bc_code = qs.QSSM_X_SOFTEDGE2
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
    # the chunk-state kernel addresses one sequence's x codes with 32-bit offsets, over whole
    # chunks plus the one its loads run ahead into: (ceil(L / 256) + 1) * 256 * nh * 64 < 2^31
    sd.nheads, sd.ngroups, sd.batch = 1 << 14, 1, 1
    sd.seqlen = 1537  # (7 + 1) * 256 * 2^14 * 64 = 2^31
    assert lib.qssm_ssd_chunk_int8(ctypes.byref(sd), None, 0, None) == qs.QSSM_ERR_UNSUPPORTED
    assert b"2^31" in lib.qssm_last_error()
    sd.seqlen = 1536  # (6 + 1) * 256 * 2^14 * 64 < 2^31: refused later, for the null pointers
    assert lib.qssm_ssd_chunk_int8(ctypes.byref(sd), None, 0, None) == qs.QSSM_ERR_INVALID_ARG
    # the workspace size covers the fp16 chunk states, their factors and the staged tables
    sd.nheads, sd.ngroups, sd.seqlen, sd.batch = 4, 1, 600, 2
    nc, nh = 3, 4
    # workspace: the fp16 state entering each chunk, per-channel x scales, per-chunk decay sums
    assert lib.qssm_ssd_workspace_size(ctypes.byref(sd)) >= (
        2 * nc * nh * 64 * 128 * 2 + nh * 64 * 4 + 2 * nc * nh * 256 * 4)


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
    """The fp32 thresholds and the fp64 EMA state, bit for bit, over many sample sizes (the
    interpolation position (n - 1) q and each rounding of the blend must agree)."""
    r = np.random.default_rng(9)
    v1 = r.standard_t(3, 100001).astype(np.float32)
    v2 = (r.standard_normal(77777) * 2).astype(np.float32)
    s, L, H, st = qs.qssm_calib_softedge(v1)
    os_, oL, oH, ost = oracle.softedge_thresholds(v1)
    assert (s, L, H) == (os_, oL, oH) and tuple(st) == ost
    s2, L2, H2, st2 = qs.qssm_calib_softedge(v2, ema_state=st)
    os2, oL2, oH2, ost2 = oracle.softedge_thresholds(v2, prev=ost)
    assert (s2, L2, H2) == (os2, oL2, oH2) and tuple(st2) == ost2
    for seed in range(60):
        r = np.random.default_rng(100 + seed)
        v = (r.standard_t(3, int(r.integers(1, 20000))) * np.exp(r.uniform(-3, 3))).astype(np.float32)
        _, _, _, st = qs.qssm_calib_softedge(v)
        assert tuple(st) == oracle.softedge_thresholds(v)[3], v.size


def test_group_and_block_absmax():
    r = np.random.default_rng(10)
    a = np.abs(r.standard_normal(300)).astype(np.float32)
    g = r.integers(0, 7, 300).astype(np.uint8)
    got = qs.qssm_calib_group_absmax(a, g, 9)
    for k in range(9):
        sel = a[g == k]
        assert got[k] == (sel.max() if sel.size else 0.0)
    assert np.array_equal(qs.qssm_calib_block_absmax(a, 4), a.reshape(75, 4).max(axis=1))
    with pytest.raises(qs.QssmError, match="below G"):
        qs.qssm_calib_group_absmax(a, g, 5)
    with pytest.raises(qs.QssmError, match="divide"):
        qs.qssm_calib_block_absmax(a, 7)


def test_layer_calibrations_match_oracle():
    """The workload drivers' calibration (library helpers) equals the oracle's, bit for bit: the
    Mamba1 x groups and B/C state groups, the SSD head-block x groups, the int8 output groups."""
    import oracle.pipelines as op
    import quantized_state_space_amd.workloads as wl
    inp = synth.mamba1_inputs(cfg=81, batch=1, seqlen=200, dim=192, dstate=16, x_dist="student_t",
                              calib_batch=2)
    p1, g1, s1 = wl.calib_x_groups(inp["x_cal"], 8)
    p2, g2, s2 = op.calib_x(inp["x_cal"], 8)
    assert np.array_equal(p1, p2) and np.array_equal(g1, g2) and np.array_equal(s1, s2)
    assert np.array_equal(wl.calib_state_groups(inp["B_cal"], 4),
                          oracle.state_group_scales(inp["B_cal"], 4))
    x = synth.rng(82, 0).standard_normal((300, 8, 64)).astype(np.float32) * \
        np.exp(synth.rng(82, 1).uniform(-2, 2, (8, 64))).astype(np.float32)
    ga, sa = wl.calib_ssd_x_groups(x, 8, 64, 2, 8)
    gb, sb = op.calib_ssd_x(x, 8, 64, 2, 8)
    assert np.array_equal(ga, gb) and np.array_equal(sa, sb)
    yg, ys = wl.calib_y_groups(inp["x_cal"], 5)
    absmax = oracle.finite_absmax(inp["x_cal"], axis=(0, 2))
    perm, grp = oracle.cluster_channels(absmax, 5)
    want_g = np.empty(absmax.size, np.uint8)
    want_g[perm] = grp
    want_s = oracle.group_scales(inp["x_cal"], want_g, 5)
    assert np.array_equal(yg, want_g) and np.array_equal(ys, want_s)


def test_s4d_state_scale_bounds_the_fp64_state():
    """The int16 state scale from the quantized parameters bounds the fp64 state of the oracle's
    run: with headroom 1, max |Re h|, |Im h| of every channel <= 32767 * scale; and the scale
    follows the stated formula (evaluated here in numpy)."""
    import oracle.pipelines as op
    inp = synth.s4d_inputs(cfg=2, batch=4, seqlen=300, channels=12, dstate=64)
    ref = op.s4d(inp)
    c, sc = ref["codes"], ref["scales"]
    umax = (np.float32(ref["su"]) * np.float32(ref["sw"]) * np.float32(128.0) *
            np.abs(ref["wq"].astype(np.float32))).astype(np.float32)
    L = inp["u"].shape[1]
    got = qs.qssm_calib_s4d_state_scale(L, c["A_re"], sc["A_re"], c["B_re"], sc["B_re"], c["B_im"],
                                        sc["B_im"], inp["log_dt"], umax, headroom=1.0)
    actual = op.s4d_state_scale(inp, headroom=1.0) * 32767.0    # max |part| of the fp64 state
    assert np.all(actual <= got.astype(np.float64) * 32767.0 * (1 + 1e-6))
    dt = np.exp(inp["log_dt"].astype(np.float64))[:, None]
    are = sc["A_re"].astype(np.float64)[:, None] * c["A_re"]
    bb = np.hypot(sc["B_re"].astype(np.float64)[:, None] * c["B_re"],
                  sc["B_im"].astype(np.float64)[:, None] * c["B_im"])
    ab = np.exp(dt * are)
    geo = np.where(ab < 1, np.minimum(1 / np.maximum(1 - ab, 1e-300), L), L * ab ** (L - 1))
    want = (dt * bb * np.maximum(ab, 1) * umax.astype(np.float64)[:, None] * geo).max(axis=1) / 32767
    np.testing.assert_allclose(got, want.astype(np.float32), rtol=1e-6)


def unpack_w4(packed, K):
    """Codes [N, K] from the packed layout (each 8 input channels in 4 bytes, byte b = code k0 + b
    in the low nibble and k0 + 4 + b in the high nibble)."""
    p = np.asarray(packed, np.uint8).reshape(packed.shape[0], K // 8, 4)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    return np.concatenate([lo, hi], axis=2).reshape(packed.shape[0], K).astype(np.int8)


def test_w4_packing_golden():
    """tests/golden/w4_packing.txt: a hand-worked example of the codes and the byte layout."""
    rows = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "w4_packing.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            rows[k] = v
    w = np.array([[float(t) for t in rows["w"]]], np.float32)
    s, packed = qs.qssm_quant_w4(w, 8)
    assert s[0, 0] == np.float32(float(rows["scale"][0]))
    assert packed[0].tolist() == [int(t, 16) for t in rows["bytes"]]
    codes = [int(t) for t in rows["codes"]]
    assert unpack_w4(packed, 8)[0].tolist() == codes
    assert oracle.quant_w4(w, 8, oracle.w4_scales(w, 8))[0].tolist() == codes


@pytest.mark.parametrize("N,K,group,seed", [(5, 64, 64, 0), (17, 256, 64, 1), (3, 128, 8, 2)])
def test_w4_quantizer_matches_oracle(N, K, group, seed):
    r = np.random.default_rng(seed)
    w = (r.standard_normal((N, K)) * np.exp(r.uniform(-3, 3, (N, 1)))).astype(np.float32)
    w[0, :4] = [np.nan, np.inf, -np.inf, 0.0]
    w[1, :group] = 0.0  # an all-zero group: scale 1, codes 0
    s, packed = qs.qssm_quant_w4(w, group)
    ws = oracle.w4_scales(w, group)
    assert np.array_equal(s, ws)
    assert np.array_equal(unpack_w4(packed, K), oracle.quant_w4(w, group, ws))
    with pytest.raises(qs.QssmError, match="group"):
        qs.qssm_quant_w4(w, 12)
