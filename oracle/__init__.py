"""Oracle for the quantized state-space hot path — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct CPU reference in fp64 (C in ``qssm_oracle.c`` plus numpy glue here).
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it. It shares no code with the HIP library ``quantized_state_space_amd`` and never imports it.

Sources (page title, section):
  Quamba2 (Chiang et al.), abstract and method steps 1-4: per-group x scales over sorted and
    clustered channels, per-state-group B/C scales, offline rearrangement, W8A8 recurrence.
  "Quantizing Small-Scale State-Space Models for Edge AI", abstract: the quantized S4D layer.
  SSDi8 abstract: the chunked SSD form with an INT8 path, persistent int8 outputs and a
    per-channel error-correction term.
  Quamba-SE soft-edge blog, sections 2.1, 2.2 and 4.1: three-scale code, byte layout, thresholds.

Every function here is pinned by a test in ``tests/test_oracle_*.py`` against something other
than itself (closed forms, special cases, brute force, library routines, error bounds).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-std=c11", "-Wall"]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _declare(_lib)
    return _lib


def max_threads() -> int:
    """OpenMP threads of the oracle's parallel loops (independent chains only)."""
    f = lib().orc_max_threads
    f.restype = ctypes.c_int
    return int(f())


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_D = ctypes.c_double
_F = ctypes.c_float


def _declare(L):
    L.orc_quant_code.argtypes = [_F, _F]
    L.orc_quant_code.restype = _I32
    L.orc_quant_group_x.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P]
    L.orc_quant_state_group.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P]
    L.orc_scale_from_absmax.argtypes = [_F]
    L.orc_scale_from_absmax.restype = _F
    L.orc_softedge_code.argtypes = [_F, _F, _F, _F, _I32]
    L.orc_softedge_code.restype = ctypes.c_uint8
    L.orc_softedge_value.argtypes = [ctypes.c_uint8, _F, _I32]
    L.orc_softedge_value.restype = _D
    L.orc_softedge_decode_f32.argtypes = [ctypes.c_uint8, _F, _I32]
    L.orc_softedge_decode_f32.restype = _F
    L.orc_softedge_encode.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I32, _P]
    L.orc_cluster_sorted.argtypes = [_P, _I32, _I32, _P]
    L.orc_selective_scan.argtypes = [_I64] * 5 + [_P] * 9
    L.orc_s4d_zoh.argtypes = [_P, _P, _D, _I64, _P, _P]
    L.orc_s4d_scan.argtypes = [_I64] * 4 + [_P] * 10
    L.orc_ssd_chunked.argtypes = [_I64] * 7 + [_P] * 7 + [_I32, _P, _P, _P, _P]
    L.orc_decode_step.argtypes = [_I64] * 5 + [_P] * 8
    L.orc_w4_scale_from_absmax.argtypes = [_F]
    L.orc_w4_scale_from_absmax.restype = _F
    L.orc_quant_w4.argtypes = [_P, _I64, _I64, _I64, _P, _P]
    L.orc_gemm_w4a8.argtypes = [_I64, _I64, _I64, _I64, _P, _F, _P, _P, _P, _P]


_KEEP = []  # arrays whose addresses were handed to C in the current call


def _ptr(a):
    if a is None:
        return None
    _KEEP.append(a)
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class _Call:
    """Keeps every converted argument alive until the C call has returned."""

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        _KEEP.clear()
        return False


# ------------------------------------------------------------------------------------------------
# Quantizer and calibration (Quamba2 steps 1-3)

def quant_code(v, s):
    """Elementwise q = clamp(RNE(v/s), -128, 127) with the exact quotient; v, s broadcastable."""
    v = np.asarray(v, dtype=np.float32)
    s = np.broadcast_to(np.asarray(s, dtype=np.float32), v.shape)
    flat_v = np.ascontiguousarray(v).reshape(-1)
    flat_s = np.ascontiguousarray(s).reshape(-1)
    out = np.empty(flat_v.shape, dtype=np.int8)
    f = lib().orc_quant_code
    for k in range(flat_v.size):
        out[k] = f(float(flat_v[k]), float(flat_s[k]))
    return out.reshape(v.shape)


def quant_group_x(x, group_of, scales, perm=None):
    """x: float32 [outer, C, inner] -> int8 codes, output channel c from input channel perm[c]."""
    x = _c(x, np.float32)
    outer, C, inner = x.shape
    q = np.empty(x.shape, dtype=np.int8)
    with _Call():
        lib().orc_quant_group_x(_ptr(x), outer, C, inner, _ptr(_c(perm, np.int32)),
                                _ptr(_c(group_of, np.uint8)), _ptr(_c(scales, np.float32)), _ptr(q))
    return q


def quant_state_group(bc, gs, scales):
    """bc: float32 [outer, Gbc, N, inner] -> int8 codes with one scale per (group, state group)."""
    bc = _c(bc, np.float32)
    outer, Gbc, N, inner = bc.shape
    q = np.empty(bc.shape, dtype=np.int8)
    with _Call():
        lib().orc_quant_state_group(_ptr(bc), outer, Gbc, N, inner, gs, _ptr(_c(scales, np.float32)),
                                    _ptr(q))
    return q


def scale_from_absmax(absmax):
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    f = lib().orc_scale_from_absmax
    return np.array([f(float(v)) for v in a], dtype=np.float32).reshape(np.shape(absmax))


def finite_absmax(x, axis):
    """Largest finite |x| along `axis` (NaN and +-Inf ignored); 0 when nothing is finite."""
    x = np.asarray(x, dtype=np.float32)
    a = np.where(np.isfinite(x), np.abs(x), np.float32(0))
    return a.max(axis=axis).astype(np.float32)


def group_scales(x, group_of, G, perm=None):
    """Per-group scales of x [outer, C, inner] after the channel permutation (fl32(absmax/127))."""
    x = np.asarray(x, dtype=np.float32)
    if perm is not None:
        x = x[:, np.asarray(perm), :]
    ch = finite_absmax(x, axis=(0, 2)) if x.size else np.zeros(x.shape[1], np.float32)
    g_abs = np.zeros(G, dtype=np.float32)
    for c, g in enumerate(np.asarray(group_of)):
        g_abs[g] = max(g_abs[g], ch[c])
    return scale_from_absmax(g_abs)


def state_group_scales(bc, gs):
    """Scales of B or C [outer, Gbc, N, inner]: one per (group, contiguous state group of gs)."""
    bc = np.asarray(bc, dtype=np.float32)
    outer, Gbc, N, inner = bc.shape
    a = finite_absmax(bc, axis=(0, 3)) if bc.size else np.zeros((Gbc, N), np.float32)
    a = a.reshape(Gbc, N // gs, gs).max(axis=2)
    return scale_from_absmax(a).reshape(-1)


def cluster_channels(absmax, G):
    """Quamba2 step 2: stable ascending sort of the channel absmax, then exact 1-D k-means (DP).

    Returns (perm, group_of): perm[c] = source channel of sorted position c, group_of[c] = group id
    of sorted position c (ascending with magnitude)."""
    absmax = np.asarray(absmax, dtype=np.float32)
    C = absmax.size
    perm = np.argsort(absmax, kind="stable").astype(np.int32)
    srt = np.ascontiguousarray(absmax[perm].astype(np.float64))
    group_of = np.empty(C, dtype=np.uint8)
    with _Call():
        lib().orc_cluster_sorted(_ptr(srt), C, G, _ptr(group_of))
    return perm, group_of


# ------------------------------------------------------------------------------------------------
# Soft-edge code (Quamba-SE 2.1, 2.2, 4.1)

SOFTEDGE_P_LOW = 5.0      # section 4.1: L at the 5th percentile
SOFTEDGE_P_HIGH = 99.9    # section 4.1: H at the 99.9th percentile
SOFTEDGE_EMA_ALPHA = 0.1  # section 4.1: EMA factor over mini-batches


def softedge_thresholds(v, alpha=SOFTEDGE_EMA_ALPHA, prev=None):
    """(s, L, H, state): L, H percentiles of |v| (numpy 'linear'), EMA-blended with prev=(L, H)
    in fp64, cast to fp32; s = fl32(H / 63). `state` is the fp64 (L, H) to pass as prev next time."""
    a = np.abs(np.asarray(v, dtype=np.float64).reshape(-1))
    l_new = float(np.percentile(a, SOFTEDGE_P_LOW))
    h_new = float(np.percentile(a, SOFTEDGE_P_HIGH))
    if prev is None:
        l, h = l_new, h_new
    else:
        l = alpha * l_new + (1.0 - alpha) * prev[0]
        h = alpha * h_new + (1.0 - alpha) * prev[1]
    L32, H32 = np.float32(l), np.float32(h)
    s = np.float32(1.0) if H32 == 0 else np.float32(H32 / np.float32(63.0))
    return s, L32, H32, (l, h)


SOFTEDGE_RATIOS = (4, 2)  # sections 2.1-2.2: scale/4 and scale*4; section 4.1: scale/2 and scale*2


def softedge_track(x, group_of, G, perm=None, alpha=SOFTEDGE_EMA_ALPHA, prev=None):
    """Per-group thresholds of one mini-batch x [outer, C, inner] in output-channel order (channel
    c reads x[:, perm[c], :] and belongs to group group_of[c]): softedge_thresholds over the group's
    values, EMA-blended with prev[g] (an fp64 (L, H) pair, or None for the first batch).
    A group with no values keeps prev[g] (or gets L = H = 0 and s = 1 without one).
    Returns s, L, H (fp32 [G]) and the new states (list of fp64 pairs)."""
    x = np.asarray(x, np.float32)
    xs = x if perm is None else x[:, np.asarray(perm, np.int64), :]
    group_of = np.asarray(group_of, np.int64)
    s = np.ones(G, np.float32)
    L = np.zeros(G, np.float32)
    H = np.zeros(G, np.float32)
    states = []
    for g in range(G):
        v = xs[:, group_of == g, :]
        p = None if prev is None else prev[g]
        if v.size == 0:
            st = (0.0, 0.0) if p is None else (float(p[0]), float(p[1]))
            L[g], H[g] = np.float32(st[0]), np.float32(st[1])
            s[g] = np.float32(1.0) if H[g] == 0 else np.float32(H[g] / np.float32(63.0))
        else:
            s[g], L[g], H[g], st = softedge_thresholds(v, alpha=alpha, prev=p)
        states.append(st)
    return s, L, H, states


def softedge_encode(x, group_of, s, L, H, perm=None, ratio=4):
    x = _c(x, np.float32)
    outer, C, inner = x.shape
    code = np.empty(x.shape, dtype=np.uint8)
    with _Call():
        lib().orc_softedge_encode(_ptr(x), outer, C, inner, _ptr(_c(perm, np.int32)),
                                  _ptr(_c(group_of, np.uint8)), _ptr(_c(s, np.float32)),
                                  _ptr(_c(L, np.float32)), _ptr(_c(H, np.float32)), int(ratio),
                                  _ptr(code))
    return code


def softedge_value_table(s, ratio=4):
    """fp64 value of each of the 256 bytes for base scale s."""
    f = lib().orc_softedge_value
    return np.array([f(b, float(s), int(ratio)) for b in range(256)], dtype=np.float64)


def softedge_values(code, group_of, s, ratio=4):
    """fp64 values of codes [outer, C, inner] (exact)."""
    code = np.asarray(code, dtype=np.uint8)
    out = np.empty(code.shape, dtype=np.float64)
    s = np.asarray(s, dtype=np.float32)
    group_of = np.asarray(group_of)
    tables = {g: softedge_value_table(s[g], ratio) for g in np.unique(group_of)}
    for c in range(code.shape[1]):
        out[:, c, :] = tables[group_of[c]][code[:, c, :]]
    return out


def softedge_decode_f32(code, group_of, s, ratio=4):
    """The library's fp32 decode: each value rounded once to fp32."""
    return softedge_values(code, group_of, s, ratio).astype(np.float32)


# ------------------------------------------------------------------------------------------------
# Dequantization (exact in fp64: an fp32 scale times an 8-bit integer)

def _usable_scales(scales):
    """fp64 scales, an invalid one (outside [2^-100, 2^100], or NaN) taken as 0: every value of
    its group is 0 (its codes are 0, and 0 * inf would be NaN)."""
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    ok = (s >= 2.0 ** -100) & (s <= 2.0 ** 100)
    return np.where(ok, s, 0.0)


def dequant_group(q, group_of, scales):
    """q [outer, C, inner] -> fp64 values scale[group_of[c]] * q."""
    s = _usable_scales(scales)[np.asarray(group_of)]
    return s[None, :, None] * np.asarray(q, dtype=np.float64)


def dequant_state_group(q, gs, scales):
    """q [outer, Gbc, N, inner] -> fp64 values."""
    outer, Gbc, N, inner = q.shape
    s = _usable_scales(scales).reshape(Gbc, N // gs)
    s = np.repeat(s, gs, axis=1)
    return s[None, :, :, None] * np.asarray(q, dtype=np.float64)


# ------------------------------------------------------------------------------------------------
# Recurrences

def selective_scan(xh, delta, A, Bh, Ch, Dskip=None, h0=None):
    """Mamba1 selective scan in fp64. xh, delta [B, D, L]; A [D, N]; Bh, Ch [B, Gbc, N, L];
    Dskip [D]; h0 [B, D, N]. Returns (y [B, D, L], h_last [B, D, N])."""
    xh = _c(xh, np.float64)
    Bsz, D, L = xh.shape
    A = _c(A, np.float64)
    N = A.shape[1]
    Bh = _c(Bh, np.float64)
    Gbc = Bh.shape[1]
    y = np.empty((Bsz, D, L), dtype=np.float64)
    h_last = np.empty((Bsz, D, N), dtype=np.float64)
    with _Call():
        lib().orc_selective_scan(Bsz, L, D, N, Gbc, _ptr(xh), _ptr(_c(delta, np.float64)), _ptr(A),
                                 _ptr(Bh), _ptr(_c(Ch, np.float64)), _ptr(_c(Dskip, np.float64)),
                                 _ptr(_c(h0, np.float64)), _ptr(y), _ptr(h_last))
    return y, h_last


def s4d_zoh(Ah, Bh, dt):
    """Zero-order hold for one channel: Ah, Bh complex [N]; returns (Abar, Bbar) complex."""
    Ah = np.ascontiguousarray(np.asarray(Ah, dtype=np.complex128))
    Bh = np.ascontiguousarray(np.asarray(Bh, dtype=np.complex128))
    Ab = np.empty_like(Ah)
    Bb = np.empty_like(Ah)
    with _Call():
        lib().orc_s4d_zoh(_ptr(Ah.view(np.float64)), _ptr(Bh.view(np.float64)), float(dt), Ah.size,
                          _ptr(Ab.view(np.float64)), _ptr(Bb.view(np.float64)))
    return Ab, Bb


def s4d_scan(u, Ah, Bh, Ch, dt, Dskip=None, state_scale=None, h0=None):
    """S4D diagonal LTI scan in fp64. u [B, H, L] real; Ah, Bh, Ch [H, N] complex; dt [H].
    Returns (y [B, H, L], h_last [B, H, N] complex)."""
    u = _c(u, np.float64)
    Bsz, H, L = u.shape
    N = np.asarray(Ah).shape[1]
    cz = lambda a: np.ascontiguousarray(np.asarray(a, dtype=np.complex128))
    Ah, Bh, Ch = cz(Ah), cz(Bh), cz(Ch)
    h0c = None if h0 is None else cz(h0)
    y = np.empty((Bsz, H, L), dtype=np.float64)
    hl = np.empty((Bsz, H, N), dtype=np.complex128)
    with _Call():
        lib().orc_s4d_scan(Bsz, L, H, N, _ptr(u), _ptr(Ah.view(np.float64)),
                           _ptr(Bh.view(np.float64)), _ptr(Ch.view(np.float64)),
                           _ptr(_c(dt, np.float64)), _ptr(_c(Dskip, np.float64)),
                           _ptr(_c(state_scale, np.float64)),
                           _ptr(None if h0c is None else h0c.view(np.float64)), _ptr(y),
                           _ptr(hl.view(np.float64)))
    return y, hl


def ssd_chunked(xh, delta, A, Bh, Ch, chunk, Dskip=None, h0=None, int8_state=False, qx=None,
                sx=None, int8_intra=False):
    """Mamba2 SSD chunked form in fp64. xh [B, L, nh, P]; delta [B, L, nh]; A [nh];
    Bh, Ch [B, L, Gbc, N]; h0 [B, nh, P, N]. int8_state=True selects the requantized chunk state
    (needs the codes qx [B, L, nh, P] and per-channel scales sx [nh*P]); that mode is exact in its
    special case (integral weighted codes) and otherwise pinned by its requantization error bound
    and the absence of rounding bias. int8_intra=True selects the int8 intra-chunk output (each
    row of the intra-chunk weights requantized with its own max / 127 scale, times the x codes;
    same inputs), pinned the same way.
    Returns (y [B, L, nh, P], h_last [B, nh, P, N])."""
    xh = _c(xh, np.float64)
    Bsz, L, nh, P = xh.shape
    Bh = _c(Bh, np.float64)
    Gbc, N = Bh.shape[2], Bh.shape[3]
    y = np.empty(xh.shape, dtype=np.float64)
    hl = np.empty((Bsz, nh, P, N), dtype=np.float64)
    with _Call():
        lib().orc_ssd_chunked(Bsz, L, nh, P, N, Gbc, chunk, _ptr(xh), _ptr(_c(delta, np.float64)),
                              _ptr(_c(A, np.float64)), _ptr(Bh), _ptr(_c(Ch, np.float64)),
                              _ptr(_c(Dskip, np.float64)), _ptr(_c(h0, np.float64)),
                              (1 if int8_state else 0) | (2 if int8_intra else 0),
                              _ptr(_c(qx, np.int8)), _ptr(_c(sx, np.float64)),
                              _ptr(y), _ptr(hl))
    return y, hl


def ssd_as_sequential(xh, delta, A, Bh, Ch, Dskip=None, h0=None):
    """The SSD layer computed by the plain sequential selective scan (A[h] shared by all (p, n)
    of head h). Same layouts as ssd_chunked; pure relayout around selective_scan."""
    xh = np.asarray(xh, dtype=np.float64)
    Bsz, L, nh, P = xh.shape
    Bh = np.asarray(Bh, dtype=np.float64)
    Gbc, N = Bh.shape[2], Bh.shape[3]
    x_s = xh.reshape(Bsz, L, nh * P).transpose(0, 2, 1)
    d_s = np.repeat(np.asarray(delta, dtype=np.float64), P, axis=2).transpose(0, 2, 1)
    A_s = np.repeat(np.asarray(A, dtype=np.float64), P)[:, None] * np.ones((1, N))
    B_s = Bh.transpose(0, 2, 3, 1)
    C_s = np.asarray(Ch, dtype=np.float64).transpose(0, 2, 3, 1)
    D_s = None if Dskip is None else np.repeat(np.asarray(Dskip, dtype=np.float64), P)
    h_s = None if h0 is None else np.asarray(h0, dtype=np.float64).reshape(Bsz, nh * P, N)
    y, hl = selective_scan(x_s, d_s, A_s, B_s, C_s, D_s, h_s)
    return y.transpose(0, 2, 1).reshape(Bsz, L, nh, P), hl.reshape(Bsz, nh, P, N)


def decode_step(xh, Bh, Ch, delta, A, state, Dskip=None):
    """One generation step. xh [B, nh, P]; Bh, Ch [B, Gbc, N]; delta [B, nh]; A [nh];
    state [B, nh, P, N] fp64, updated in place. Returns y [B, nh, P]."""
    xh = _c(xh, np.float64)
    Bsz, nh, P = xh.shape
    Bh = _c(Bh, np.float64)
    Gbc, N = Bh.shape[1], Bh.shape[2]
    assert state.dtype == np.float64 and state.flags.c_contiguous
    y = np.empty((Bsz, nh, P), dtype=np.float64)
    with _Call():
        lib().orc_decode_step(Bsz, nh, P, N, Gbc, _ptr(xh), _ptr(Bh), _ptr(_c(Ch, np.float64)),
                              _ptr(_c(delta, np.float64)), _ptr(_c(A, np.float64)),
                              _ptr(_c(Dskip, np.float64)), _ptr(state), _ptr(y))
    return y


# ------------------------------------------------------------------------------------------------
# W4A8 linear layer (Quamba2 abstract: W4A8 for large-batch decoding). 4-bit symmetric weights with
# a scale per (output channel, group of input channels), int8 activations with one scale.

def w4_scales(w, group):
    """Scales [N, K / group]: fl32(absmax / 7) of each group of `group` consecutive input channels
    (absmax 0 -> 1, clamped into [2^-100, 2^100])."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    a = finite_absmax(w.reshape(N, K // group, group), axis=2)
    f = lib().orc_w4_scale_from_absmax
    return np.array([f(float(v)) for v in a.reshape(-1)], np.float32).reshape(N, K // group)


def quant_w4(w, group, scales):
    """Codes [N, K] in [-8, 7]: clamp(RNE(w / s), -8, 7) with the exact quotient (int8 storage)."""
    w = _c(w, np.float32)
    N, K = w.shape
    q = np.empty((N, K), np.int8)
    with _Call():
        lib().orc_quant_w4(_ptr(w), N, K, group, _ptr(_c(scales, np.float32)), _ptr(q))
    return q


def gemm_w4a8(qa, sa, qw, sw, group, bias=None):
    """y [M, N] in fp64: bias[n] + sum_g sa sw[n, g] sum_{k in g} qa[m, k] qw[n, k]."""
    qa = _c(qa, np.int8)
    qw = _c(qw, np.int8)
    M, K = qa.shape
    N = qw.shape[0]
    y = np.empty((M, N), np.float64)
    with _Call():
        lib().orc_gemm_w4a8(M, N, K, group, _ptr(qa), float(np.float32(sa)), _ptr(qw),
                            _ptr(_c(sw, np.float32)), _ptr(_c(bias, np.float64)), _ptr(y))
    return y


# ------------------------------------------------------------------------------------------------
# Persistent int8 output (SSDi8 abstract: the layer hands the next W8A8 module int8 activations,
# and an error-correction term from per-channel error statistics)

def requant_output(y, group_of, scales, bias=None):
    """Int8 codes of a layer output y [outer, C, inner] for the next W8A8 module: the per-channel
    correction bias[c] is added, then channel c is quantized with scales[group_of[c]] by the
    int8 rule (exact quotient, round half to even, saturation, an invalid scale gives 0).
    The decision is taken in fp32, the precision the output is produced in: v = fl32(fl32(y) +
    bias[c]), then the exact quotient v / s."""
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    outer, C, inner = y32.shape
    b = np.zeros(C, np.float32) if bias is None else np.asarray(bias, dtype=np.float32)
    v = (y32 + b[None, :, None]).astype(np.float32)
    s = np.asarray(scales, dtype=np.float32)[np.asarray(group_of, dtype=np.int64)]
    return quant_code(v, np.broadcast_to(s[None, :, None], v.shape))


def channel_error_mean(ref, approx):
    """Per-channel error statistic of a quantized path: mean over outer and inner of ref - approx,
    for [outer, C, inner] arrays, accumulated in fp64 (the correction term's calibration)."""
    d = np.asarray(ref, dtype=np.float64) - np.asarray(approx, dtype=np.float64)
    return d.mean(axis=(0, 2))


# ------------------------------------------------------------------------------------------------
# Output comparison rule

def rowwise_error(y, ref, axis=-1):
    """Per-row normwise error: max|y - r| / max(max|r|, 1e-6 * max_all|r|) along `axis`.
    Complex inputs (the S4D state) use the modulus. Returns the array of per-row errors."""
    dt = np.complex128 if (np.iscomplexobj(y) or np.iscomplexobj(ref)) else np.float64
    y = np.asarray(y, dtype=dt)
    ref = np.asarray(ref, dtype=dt)
    floor = 1e-6 * max(np.abs(ref).max(initial=0.0), 1e-300)
    num = np.abs(y - ref).max(axis=axis)
    den = np.maximum(np.abs(ref).max(axis=axis), floor)
    return num / den
