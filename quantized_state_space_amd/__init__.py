"""Python binding of libqssm (ctypes): the C entry points under the same names.

Argument marshalling only: every step of the hot path runs in the library's HIP kernels. Tensors
are torch tensors on the GPU (PyTorch provides device memory and streams); they are checked for
dtype, device and contiguity and passed as raw pointers with the current HIP stream. There is no
fallback: if ``libqssm.so`` is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqssm.so")

QSSM_OK, QSSM_ERR_INVALID_ARG, QSSM_ERR_UNSUPPORTED, QSSM_ERR_WORKSPACE, QSSM_ERR_DEVICE = range(5)
QSSM_F32, QSSM_F16, QSSM_I16, QSSM_I8 = 0, 1, 2, 3
QSSM_X_INT8, QSSM_X_SOFTEDGE, QSSM_X_SOFTEDGE2 = 0, 1, 2
QSSM_MMA_F16, QSSM_MMA_I8 = 0, 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


class QssmError(RuntimeError):
    def __init__(self, name, status, message):
        super().__init__(f"{name} failed with status {status}: {message}")
        self.status = status


class ScanArgs(ctypes.Structure):
    _fields_ = [("batch", _I64), ("seqlen", _I64), ("dim", _I64), ("dstate", _I64),
                ("x_code", _I32), ("x_groups", _I32), ("x", _P), ("x_group_of", _P),
                ("x_scales", _P), ("delta", _P), ("A", _P), ("bc_groups", _I32),
                ("bc_group_size", _I32), ("Bq", _P), ("Cq", _P), ("B_scales", _P), ("C_scales", _P),
                ("Dskip", _P), ("h0", _P), ("y", _P), ("y_dtype", _I32), ("h_last", _P),
                ("y_groups", _I32), ("y_group_of", _P), ("y_scales", _P), ("y_bias", _P),
                ("bc_code", _I32), ("time_blocks", _I32)]


class S4dArgs(ctypes.Structure):
    _fields_ = [("batch", _I64), ("seqlen", _I64), ("channels", _I64), ("dstate", _I64),
                ("uq", _P), ("u_scale", _P), ("wq", _P), ("w_scale", _P),
                ("A_re", _P), ("A_im", _P), ("B_re", _P), ("B_im", _P), ("C_re", _P), ("C_im", _P),
                ("A_re_s", _P), ("A_im_s", _P), ("B_re_s", _P), ("B_im_s", _P), ("C_re_s", _P),
                ("C_im_s", _P), ("log_dt", _P), ("Dskip", _P), ("state_dtype", _I32),
                ("state_scale", _P), ("h0", _P), ("y", _P), ("h_last", _P)]


class SsdArgs(ctypes.Structure):
    _fields_ = [("batch", _I64), ("seqlen", _I64), ("nheads", _I64), ("headdim", _I64),
                ("dstate", _I64), ("ngroups", _I32), ("chunk", _I32), ("x_groups", _I32),
                ("xq", _P), ("x_group_of", _P), ("x_scales", _P), ("delta", _P), ("A", _P),
                ("Dskip", _P), ("bc_group_size", _I32), ("Bq", _P), ("Cq", _P), ("B_scales", _P),
                ("C_scales", _P), ("h0", _P), ("y", _P), ("y_dtype", _I32), ("h_last", _P),
                ("fused", _I32), ("state_mma", _I32), ("y_groups", _I32), ("y_group_of", _P),
                ("y_scales", _P), ("y_bias", _P), ("intra_mma", _I32)]


class UpdateArgs(ctypes.Structure):
    _fields_ = [("batch", _I64), ("nheads", _I64), ("headdim", _I64), ("dstate", _I64),
                ("ngroups", _I32), ("x_groups", _I32), ("x", _P), ("x_group_of", _P),
                ("x_scales", _P), ("B", _P), ("C", _P), ("bc_group_size", _I32),
                ("B_scales", _P), ("C_scales", _P), ("delta", _P), ("A", _P), ("Dskip", _P),
                ("state_dtype", _I32), ("state", _P), ("y", _P), ("xq_out", _P), ("Bq_out", _P),
                ("Cq_out", _P), ("y_dtype", _I32), ("y_groups", _I32), ("y_group_of", _P),
                ("y_scales", _P), ("y_bias", _P)]


class GemmArgs(ctypes.Structure):
    _fields_ = [("M", _I64), ("N", _I64), ("K", _I64), ("group", _I32), ("y_dtype", _I32),
                ("a", _P), ("a_scale", _P), ("w", _P), ("w_scales", _P), ("bias", _P), ("y", _P)]


ARG_STRUCTS = {0: ScanArgs, 1: S4dArgs, 2: SsdArgs, 3: UpdateArgs, 4: GemmArgs}

# Every symbol include/qssm.h declares, with its ctypes signature.
SIGNATURES = {
    "qssm_quant_group_x": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I32, _P, _I32, _P, _P]),
    "qssm_quant_state_group_BC": (_I32, [_P, _I64, _I32, _I32, _I64, _I32, _P, _I32, _P, _P]),
    "qssm_softedge_encode": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I32, _P, _P, _P, _I32, _P, _P]),
    "qssm_softedge_decode": (_I32, [_P, _I64, _I64, _I64, _P, _I32, _P, _I32, _P, _P]),
    "qssm_softedge_track_workspace_size": (ctypes.c_size_t, [_I32]),
    "qssm_probe_rate": (_I32, [_I32, _I64, _I32, _P, _P]),
    "qssm_softedge_track": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I32, ctypes.c_double, _I32, _P,
                                   _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "qssm_scan_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(ScanArgs)]),
    "qssm_scan_w8a8": (_I32, [ctypes.POINTER(ScanArgs), _P, ctypes.c_size_t, _P]),
    "qssm_scan_w8a8_noalloc": (_I32, [ctypes.POINTER(ScanArgs), _P]),
    "qssm_s4d_scan": (_I32, [ctypes.POINTER(S4dArgs), _P]),
    "qssm_ssd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(SsdArgs)]),
    "qssm_ssd_chunk_int8": (_I32, [ctypes.POINTER(SsdArgs), _P, ctypes.c_size_t, _P]),
    "qssm_state_update": (_I32, [ctypes.POINTER(UpdateArgs), _P]),
    "qssm_gemm_w4a8": (_I32, [ctypes.POINTER(GemmArgs), _P]),
    "qssm_quant_w4": (_I32, [_P, _I64, _I64, _I32, _P, _P]),
    "qssm_calib_channel_absmax": (_I32, [_P, _I64, _I64, _I64, _P]),
    "qssm_calib_scales": (_I32, [_P, _I64, _P]),
    "qssm_calib_cluster_channels": (_I32, [_P, _I32, _I32, _P, _P]),
    "qssm_calib_softedge": (_I32, [_P, _I64, ctypes.c_double, _I32, _P, _P, _P, _P]),
    "qssm_calib_channel_error_mean": (_I32, [_P, _P, _I64, _I64, _I64, _P]),
    "qssm_calib_group_absmax": (_I32, [_P, _P, _I64, _I32, _P]),
    "qssm_calib_block_absmax": (_I32, [_P, _I64, _I32, _P]),
    "qssm_calib_s4d_state_scale": (_I32, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P,
                                          ctypes.c_double, _P]),
    "qssm_status_string": (ctypes.c_char_p, [_I32]),
    "qssm_last_error": (ctypes.c_char_p, []),
    "qssm_version": (_I32, []),
    "qssm_args_size": (ctypes.c_size_t, [_I32]),
}

_lib = None


def load():
    """Load libqssm.so (built in-tree by ``__graft_entry__.build()``). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        for kind, st in ARG_STRUCTS.items():
            if lib.qssm_args_size(kind) != ctypes.sizeof(st):
                raise ImportError(f"argument struct {st.__name__} layout mismatch")
        _lib = lib
    return _lib


def _check(name, status):
    if status != QSSM_OK:
        raise QssmError(name, status, load().qssm_last_error().decode())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t, dtype=None, name="tensor", optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _t():
    import torch
    return torch


# ------------------------------------------------------------------------------------------------
# Quantizers and soft-edge code

def qssm_quant_group_x(x, group_of, G, scales, q, perm=None, compute_scales=False, stream=None):
    """x: float32 [outer, C, inner]; q: int8, same shape; scales float32 [G] (in or out)."""
    torch = _t()
    outer, C, inner = x.shape
    _check("qssm_quant_group_x", load().qssm_quant_group_x(
        _ptr(x, torch.float32, "x"), outer, C, inner, _ptr(perm, torch.int32, "perm", True),
        _ptr(group_of, torch.uint8, "group_of"), G, _ptr(scales, torch.float32, "scales"),
        int(bool(compute_scales)), _ptr(q, torch.int8, "q"), _stream(stream)))
    return q


def qssm_quant_state_group_BC(bc, gs, scales, q, compute_scales=False, stream=None):
    """bc: float32 [outer, Gbc, N, inner]; q int8 same shape; scales [Gbc * N / gs]."""
    torch = _t()
    outer, Gbc, N, inner = bc.shape
    _check("qssm_quant_state_group_BC", load().qssm_quant_state_group_BC(
        _ptr(bc, torch.float32, "bc"), outer, Gbc, N, inner, gs,
        _ptr(scales, torch.float32, "scales"), int(bool(compute_scales)),
        _ptr(q, torch.int8, "q"), _stream(stream)))
    return q


def qssm_softedge_encode(x, group_of, G, s, L, H, code, perm=None, form=QSSM_X_SOFTEDGE,
                         stream=None):
    torch = _t()
    outer, C, inner = x.shape
    _check("qssm_softedge_encode", load().qssm_softedge_encode(
        _ptr(x, torch.float32, "x"), outer, C, inner, _ptr(perm, torch.int32, "perm", True),
        _ptr(group_of, torch.uint8, "group_of"), G, _ptr(s, torch.float32, "s"),
        _ptr(L, torch.float32, "L"), _ptr(H, torch.float32, "H"), int(form),
        _ptr(code, torch.uint8, "code"), _stream(stream)))
    return code


def qssm_softedge_decode(code, group_of, G, s, out, form=QSSM_X_SOFTEDGE, stream=None):
    torch = _t()
    outer, C, inner = code.shape
    _check("qssm_softedge_decode", load().qssm_softedge_decode(
        _ptr(code, torch.uint8, "code"), outer, C, inner, _ptr(group_of, torch.uint8, "group_of"),
        G, _ptr(s, torch.float32, "s"), int(form), _ptr(out, torch.float32, "out"),
        _stream(stream)))
    return out


QSSM_PROBE_EXP, QSSM_PROBE_FMA, QSSM_PROBE_EXP_FMA, QSSM_PROBE_MFMA_I8, QSSM_PROBE_MFMA_F16 = range(5)


def qssm_probe_rate(kind, iters, blocks, sink, stream=None):
    """Instruction-rate loop (measurement support); sink: float32 device tensor of blocks * 256."""
    torch = _t()
    if sink.numel() < blocks * 256:
        raise ValueError("sink must hold blocks * 256 floats")
    _check("qssm_probe_rate", load().qssm_probe_rate(int(kind), int(iters), int(blocks),
                                                    _ptr(sink, torch.float32, "sink"),
                                                    _stream(stream)))


def qssm_softedge_track_workspace_size(G):
    return load().qssm_softedge_track_workspace_size(int(G))


def qssm_softedge_track(x, group_of, G, ema_state, s, L, H, workspace, ema_valid, perm=None,
                        alpha=0.1, stream=None):
    """Per-group P5 / P99.9 thresholds of x [outer, C, inner] on the device, EMA-blended with
    ema_state (float64 [G, 2], updated in place) when ema_valid; writes s, L, H (float32 [G])."""
    torch = _t()
    outer, C, inner = x.shape
    if group_of.numel() != C:
        raise ValueError("group_of must have one entry per channel")
    if ema_state.numel() != 2 * G or s.numel() != G or L.numel() != G or H.numel() != G:
        raise ValueError("ema_state must hold 2 G values and s, L, H G values each")
    _check("qssm_softedge_track", load().qssm_softedge_track(
        _ptr(x, torch.float32, "x"), outer, C, inner, _ptr(perm, torch.int32, "perm", True),
        _ptr(group_of, torch.uint8, "group_of"), int(G), float(alpha), int(bool(ema_valid)),
        _ptr(ema_state, torch.float64, "ema_state"), _ptr(s, torch.float32, "s"),
        _ptr(L, torch.float32, "L"), _ptr(H, torch.float32, "H"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


# ------------------------------------------------------------------------------------------------
# Recurrences

def _fill(st, keep=(), **kw):
    """Sets the fields of an argument struct. The struct keeps a reference to every tensor whose
    address it holds (`keep`), so temporaries passed by the caller outlive the struct."""
    for k, v in kw.items():
        setattr(st, k, v)
    st._keep = [t for t in keep if t is not None]
    return st


def scan_args(x, x_code, x_group_of, x_scales, delta, A, Bq, Cq, B_scales, C_scales, gs, y,
              Dskip=None, h0=None, h_last=None, y_group_of=None, y_scales=None, y_bias=None,
              bc_code=QSSM_X_INT8, time_blocks=0):
    """Builds ScanArgs for x [B, D, L] codes, Bq/Cq [B, Gbc, N, L] (int8, or uint8 soft-edge bytes
    when bc_code is a soft-edge form). An int8 y takes the output group map, scales and
    (optional) correction bias. time_blocks: 0 library choice, 1 chain form, K >= 2 windows."""
    torch = _t()
    B, D, L = x.shape
    N = A.shape[1]
    Gbc = Bq.shape[1]
    xdt = torch.int8 if x_code == QSSM_X_INT8 else torch.uint8
    bdt = torch.int8 if bc_code == QSSM_X_INT8 else torch.uint8
    ydt = {torch.float32: QSSM_F32, torch.float16: QSSM_F16, torch.int8: QSSM_I8}.get(y.dtype, -1)
    yq = ydt == QSSM_I8
    if yq:
        if y_group_of is None or y_scales is None:
            raise ValueError("an int8 y needs y_group_of and y_scales")
        if y_group_of.numel() != D or (y_bias is not None and y_bias.numel() != D):
            raise ValueError("y_group_of and y_bias must have one entry per channel")
    if x_group_of.numel() != D:
        raise ValueError("x_group_of must have one entry per channel")
    keep = (x, x_group_of, x_scales, delta, A, Bq, Cq, B_scales, C_scales, y, Dskip, h0, h_last,
            y_group_of, y_scales, y_bias)
    return _fill(ScanArgs(), keep=keep, batch=B, seqlen=L, dim=D, dstate=N, x_code=x_code,
                 y_groups=int(y_scales.numel()) if (yq and y_scales is not None) else 0,
                 y_group_of=_ptr(y_group_of, torch.uint8, "y_group_of", not yq),
                 y_scales=_ptr(y_scales, torch.float32, "y_scales", not yq),
                 y_bias=_ptr(y_bias, torch.float32, "y_bias", True),
                 x_groups=int(x_scales.numel()), x=_ptr(x, xdt, "x"),
                 x_group_of=_ptr(x_group_of, torch.uint8, "x_group_of"),
                 x_scales=_ptr(x_scales, torch.float32, "x_scales"),
                 delta=_ptr(delta, torch.float32, "delta"), A=_ptr(A, torch.float32, "A"),
                 bc_groups=Gbc, bc_group_size=gs, bc_code=int(bc_code), time_blocks=int(time_blocks),
                 Bq=_ptr(Bq, bdt, "Bq"),
                 Cq=_ptr(Cq, bdt, "Cq"), B_scales=_ptr(B_scales, torch.float32, "B_scales"),
                 C_scales=_ptr(C_scales, torch.float32, "C_scales"),
                 Dskip=_ptr(Dskip, torch.float32, "Dskip", True),
                 h0=_ptr(h0, torch.float32, "h0", True), y=_ptr(y, None, "y"), y_dtype=ydt,
                 h_last=_ptr(h_last, torch.float32, "h_last", True))


def qssm_scan_workspace_size(args):
    return load().qssm_scan_workspace_size(ctypes.byref(args))


def qssm_scan_w8a8(args, workspace, stream=None):
    torch = _t()
    _check("qssm_scan_w8a8", load().qssm_scan_w8a8(
        ctypes.byref(args), _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream)))


# Size of the library-owned staging array used by qssm_scan_w8a8_noalloc (QSSM_SCAN_SCRATCH_BYTES).
QSSM_SCAN_SCRATCH_BYTES = 32 << 20


def qssm_scan_w8a8_noalloc(args, stream=None):
    """The scan without a caller workspace (the library's fixed staging array; calls on one GPU
    must not overlap)."""
    _check("qssm_scan_w8a8_noalloc", load().qssm_scan_w8a8_noalloc(ctypes.byref(args),
                                                                    _stream(stream)))


def s4d_args(uq, u_scale, params, scales, log_dt, y, wq=None, w_scale=None, Dskip=None,
             state_dtype=QSSM_F32, state_scale=None, h0=None, h_last=None, channels=None):
    """params: dict of int8 [H, N] planes A_re, A_im, B_re, B_im, C_re, C_im;
    scales: dict of float32 [H] with the same keys."""
    torch = _t()
    H, N = params["A_re"].shape
    B = uq.shape[0]
    L = uq.shape[-1]
    kw = {k: _ptr(params[k], torch.int8, k) for k in ("A_re", "A_im", "B_re", "B_im", "C_re", "C_im")}
    kw.update({k + "_s": _ptr(scales[k], torch.float32, k + "_s")
               for k in ("A_re", "A_im", "B_re", "B_im", "C_re", "C_im")})
    st_t = torch.float32 if state_dtype == QSSM_F32 else torch.int16
    keep = (uq, u_scale, log_dt, y, wq, w_scale, Dskip, state_scale, h0, h_last,
            *params.values(), *scales.values())
    return _fill(S4dArgs(), keep=keep, batch=B, seqlen=L, channels=H, dstate=N, uq=_ptr(uq, torch.int8, "uq"),
                 u_scale=_ptr(u_scale, torch.float32, "u_scale"), wq=_ptr(wq, torch.int8, "wq", True),
                 w_scale=_ptr(w_scale, torch.float32, "w_scale", True),
                 log_dt=_ptr(log_dt, torch.float32, "log_dt"),
                 Dskip=_ptr(Dskip, torch.float32, "Dskip", True), state_dtype=state_dtype,
                 state_scale=_ptr(state_scale, torch.float32, "state_scale", True),
                 h0=_ptr(h0, st_t, "h0", True), y=_ptr(y, torch.float32, "y"),
                 h_last=_ptr(h_last, st_t, "h_last", True), **kw)


def qssm_s4d_scan(args, stream=None):
    _check("qssm_s4d_scan", load().qssm_s4d_scan(ctypes.byref(args), _stream(stream)))


def _y_out_fields(y, nch, y_group_of, y_scales, y_bias):
    """The int8-output fields of an argument block (y is int8), checked for size."""
    torch = _t()
    yq = y.dtype == torch.int8
    if yq:
        if y_group_of is None or y_scales is None:
            raise ValueError("an int8 y needs y_group_of and y_scales")
        if y_group_of.numel() != nch or (y_bias is not None and y_bias.numel() != nch):
            raise ValueError("y_group_of and y_bias must have one entry per channel")
    return dict(y_groups=int(y_scales.numel()) if yq else 0,
                y_group_of=_ptr(y_group_of, torch.uint8, "y_group_of", not yq),
                y_scales=_ptr(y_scales, torch.float32, "y_scales", not yq),
                y_bias=_ptr(y_bias, torch.float32, "y_bias", True))


def ssd_args(xq, x_group_of, x_scales, delta, A, Bq, Cq, B_scales, C_scales, gs, chunk, y,
             Dskip=None, h0=None, h_last=None, state_mma=QSSM_MMA_F16, y_group_of=None,
             y_scales=None, y_bias=None, intra_mma=QSSM_MMA_F16):
    """y is float32, float16 or int8 (then y_group_of [nh * P], y_scales [Gy] and the optional
    correction y_bias [nh * P] are given)."""
    torch = _t()
    B, L, nh, P = xq.shape
    Gbc, N = Bq.shape[2], Bq.shape[3]
    ydt = {torch.float32: QSSM_F32, torch.float16: QSSM_F16, torch.int8: QSSM_I8}.get(y.dtype, -1)
    keep = (xq, x_group_of, x_scales, delta, A, Bq, Cq, B_scales, C_scales, y, Dskip, h0, h_last,
            y_group_of, y_scales, y_bias)
    return _fill(SsdArgs(), keep=keep, **_y_out_fields(y, nh * P, y_group_of, y_scales, y_bias),
                 batch=B, seqlen=L, nheads=nh, headdim=P, dstate=N, ngroups=Gbc,
                 chunk=chunk, x_groups=int(x_scales.numel()), xq=_ptr(xq, torch.int8, "xq"),
                 x_group_of=_ptr(x_group_of, torch.uint8, "x_group_of"),
                 x_scales=_ptr(x_scales, torch.float32, "x_scales"),
                 delta=_ptr(delta, torch.float32, "delta"), A=_ptr(A, torch.float32, "A"),
                 Dskip=_ptr(Dskip, torch.float32, "Dskip", True), bc_group_size=gs,
                 Bq=_ptr(Bq, torch.int8, "Bq"), Cq=_ptr(Cq, torch.int8, "Cq"),
                 B_scales=_ptr(B_scales, torch.float32, "B_scales"),
                 C_scales=_ptr(C_scales, torch.float32, "C_scales"),
                 h0=_ptr(h0, torch.float32, "h0", True), y=_ptr(y, None, "y"), y_dtype=ydt,
                 h_last=_ptr(h_last, torch.float32, "h_last", True), fused=0,
                 state_mma=state_mma, intra_mma=intra_mma)


def qssm_ssd_workspace_size(args):
    return load().qssm_ssd_workspace_size(ctypes.byref(args))


def qssm_ssd_chunk_int8(args, workspace, stream=None):
    torch = _t()
    _check("qssm_ssd_chunk_int8", load().qssm_ssd_chunk_int8(
        ctypes.byref(args), _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream)))


def update_args(x, x_group_of, x_scales, Bm, Cm, B_scales, C_scales, gs, delta, A, state, y,
                Dskip=None, xq_out=None, Bq_out=None, Cq_out=None, y_group_of=None,
                y_scales=None, y_bias=None):
    """y is float32 or int8 (then y_group_of [nh * P], y_scales [Gy] and the optional correction
    y_bias [nh * P] are given)."""
    torch = _t()
    B, nh, P = x.shape
    Gbc, N = Bm.shape[1], Bm.shape[2]
    sdt = QSSM_F32 if state.dtype == torch.float32 else QSSM_F16
    keep = (x, x_group_of, x_scales, Bm, Cm, B_scales, C_scales, delta, A, state, y, Dskip, xq_out,
            Bq_out, Cq_out, y_group_of, y_scales, y_bias)
    ydt = {torch.float32: QSSM_F32, torch.int8: QSSM_I8}.get(y.dtype, -1)
    return _fill(UpdateArgs(), keep=keep, **_y_out_fields(y, nh * P, y_group_of, y_scales, y_bias),
                 y_dtype=ydt, batch=B, nheads=nh, headdim=P, dstate=N, ngroups=Gbc,
                 x_groups=int(x_scales.numel()), x=_ptr(x, torch.float32, "x"),
                 x_group_of=_ptr(x_group_of, torch.uint8, "x_group_of"),
                 x_scales=_ptr(x_scales, torch.float32, "x_scales"), B=_ptr(Bm, torch.float32, "B"),
                 C=_ptr(Cm, torch.float32, "C"), bc_group_size=gs,
                 B_scales=_ptr(B_scales, torch.float32, "B_scales"),
                 C_scales=_ptr(C_scales, torch.float32, "C_scales"),
                 delta=_ptr(delta, torch.float32, "delta"), A=_ptr(A, torch.float32, "A"),
                 Dskip=_ptr(Dskip, torch.float32, "Dskip", True), state_dtype=sdt,
                 state=_ptr(state, None, "state"), y=_ptr(y, None, "y"),
                 xq_out=_ptr(xq_out, torch.int8, "xq_out", True),
                 Bq_out=_ptr(Bq_out, torch.int8, "Bq_out", True),
                 Cq_out=_ptr(Cq_out, torch.int8, "Cq_out", True))


def qssm_state_update(args, stream=None):
    _check("qssm_state_update", load().qssm_state_update(ctypes.byref(args), _stream(stream)))


# ------------------------------------------------------------------------------------------------
# W4A8 linear layer

def gemm_args(a, a_scale, w_packed, w_scales, group, y, bias=None):
    """a: int8 [M, K]; a_scale float32 [1]; w_packed uint8 [N, K / 2] (qssm_quant_w4 layout);
    w_scales float32 [N, K / group]; y float32 or float16 [M, N]; bias float32 [N] or None."""
    torch = _t()
    M, K = a.shape
    N = w_packed.shape[0]
    if tuple(w_packed.shape) != (N, K // 2) or tuple(y.shape) != (M, N):
        raise ValueError("shapes of a, w_packed and y do not match")
    if w_scales.numel() != N * (K // group) or (bias is not None and bias.numel() != N):
        raise ValueError("w_scales must be [N, K / group] and bias [N]")
    ydt = {torch.float32: QSSM_F32, torch.float16: QSSM_F16}.get(y.dtype, -1)
    keep = (a, a_scale, w_packed, w_scales, y, bias)
    return _fill(GemmArgs(), keep=keep, M=M, N=N, K=K, group=group, y_dtype=ydt,
                 a=_ptr(a, torch.int8, "a"), a_scale=_ptr(a_scale, torch.float32, "a_scale"),
                 w=_ptr(w_packed, torch.uint8, "w"),
                 w_scales=_ptr(w_scales, torch.float32, "w_scales"),
                 bias=_ptr(bias, torch.float32, "bias", True), y=_ptr(y, None, "y"))


def qssm_gemm_w4a8(args, stream=None):
    _check("qssm_gemm_w4a8", load().qssm_gemm_w4a8(ctypes.byref(args), _stream(stream)))


# ------------------------------------------------------------------------------------------------
# Host calibration (numpy arrays on the CPU)

def qssm_quant_w4(w, group):
    """Offline 4-bit weight quantization (host): returns (scales [N, K / group] float32,
    packed [N, K / 2] uint8)."""
    import numpy as np
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    scales = np.empty((N, K // group if group > 0 else 0), np.float32)
    packed = np.empty((N, K // 2), np.uint8)
    _check("qssm_quant_w4", load().qssm_quant_w4(_np_ptr(w), N, K, group, _np_ptr(scales),
                                                  _np_ptr(packed)))
    return scales, packed

def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def qssm_calib_channel_absmax(x):
    import numpy as np
    x = np.ascontiguousarray(x, dtype=np.float32)
    outer, C, inner = x.shape
    out = np.empty(C, dtype=np.float32)
    _check("qssm_calib_channel_absmax",
           load().qssm_calib_channel_absmax(_np_ptr(x), outer, C, inner, _np_ptr(out)))
    return out


def qssm_calib_scales(absmax):
    import numpy as np
    a = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    out = np.empty_like(a)
    _check("qssm_calib_scales", load().qssm_calib_scales(_np_ptr(a), a.size, _np_ptr(out)))
    return out


def qssm_calib_cluster_channels(absmax, G):
    import numpy as np
    a = np.ascontiguousarray(absmax, dtype=np.float32)
    perm = np.empty(a.size, dtype=np.int32)
    grp = np.empty(a.size, dtype=np.uint8)
    _check("qssm_calib_cluster_channels",
           load().qssm_calib_cluster_channels(_np_ptr(a), a.size, G, _np_ptr(perm), _np_ptr(grp)))
    return perm, grp


def qssm_calib_channel_error_mean(ref, approx):
    """Per-channel mean of ref - approx over axes 0 and 2 of [outer, C, inner] host arrays."""
    import numpy as np
    r = np.ascontiguousarray(ref, dtype=np.float32)
    a = np.ascontiguousarray(approx, dtype=np.float32)
    if r.shape != a.shape or r.ndim != 3:
        raise ValueError("ref and approx must be [outer, C, inner] arrays of one shape")
    outer, C, inner = r.shape
    out = np.empty(C, dtype=np.float32)
    _check("qssm_calib_channel_error_mean", load().qssm_calib_channel_error_mean(
        _np_ptr(r), _np_ptr(a), outer, C, inner, _np_ptr(out)))
    return out


def qssm_calib_softedge(v, alpha=0.1, ema_state=None):
    """Returns (s, L, H, ema_state); pass ema_state back to blend the next batch."""
    import numpy as np
    v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
    st = np.zeros(2, dtype=np.float64) if ema_state is None else np.array(ema_state, np.float64)
    s = np.zeros(1, np.float32)
    L = np.zeros(1, np.float32)
    H = np.zeros(1, np.float32)
    _check("qssm_calib_softedge", load().qssm_calib_softedge(
        _np_ptr(v), v.size, float(alpha), int(ema_state is not None), _np_ptr(st), _np_ptr(s),
        _np_ptr(L), _np_ptr(H)))
    return s[0], L[0], H[0], st


def qssm_calib_group_absmax(absmax, group_of, G):
    """Per-group maximum of channel absmax values (host arrays)."""
    import numpy as np
    a = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    g = np.ascontiguousarray(group_of, dtype=np.uint8).reshape(-1)
    if a.size != g.size:
        raise ValueError("absmax and group_of must have one entry per channel")
    out = np.empty(G, np.float32)
    _check("qssm_calib_group_absmax",
           load().qssm_calib_group_absmax(_np_ptr(a), _np_ptr(g), a.size, G, _np_ptr(out)))
    return out


def qssm_calib_block_absmax(absmax, block):
    """Maximum of each contiguous block of `block` values (host array)."""
    import numpy as np
    a = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    out = np.empty(a.size // block if block > 0 else 0, np.float32)
    _check("qssm_calib_block_absmax",
           load().qssm_calib_block_absmax(_np_ptr(a), a.size, block, _np_ptr(out)))
    return out


def qssm_calib_s4d_state_scale(L, A_re, A_re_s, B_re, B_re_s, B_im, B_im_s, log_dt, umax,
                               headroom=1.25):
    """Per-channel int16 S4D state scale from the quantized parameters (host arrays: int8 planes
    [H, N], fp32 scales [H], log_dt [H], umax [H])."""
    import numpy as np
    c8 = lambda a: np.ascontiguousarray(a, dtype=np.int8)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    planes = [c8(A_re), c8(B_re), c8(B_im)]
    H, N = planes[0].shape
    sc = [f32(A_re_s), f32(B_re_s), f32(B_im_s), f32(log_dt), f32(umax)]
    out = np.empty(H, np.float32)
    _check("qssm_calib_s4d_state_scale", load().qssm_calib_s4d_state_scale(
        H, N, L, _np_ptr(planes[0]), _np_ptr(sc[0]), _np_ptr(planes[1]), _np_ptr(sc[1]),
        _np_ptr(planes[2]), _np_ptr(sc[2]), _np_ptr(sc[3]), _np_ptr(sc[4]), float(headroom),
        _np_ptr(out)))
    return out
