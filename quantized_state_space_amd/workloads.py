"""Workload drivers of the hot path: calibration with the library's host helpers, device buffers,
and one call sequence per layer type. Orchestration only: every arithmetic step runs in libqssm
(host calibration in its C++ helpers, everything else in its HIP kernels); torch only allocates
device memory and provides the stream.

Channel rearrangement (Quamba2, method step 4): the x channels are gathered into cluster order by
the quantizer (perm); delta, A and D are stored in the same order, as the offline-rearranged weights
that produce them would emit them.
"""
from __future__ import annotations

import numpy as np

from . import (QSSM_F16, QSSM_F32, QSSM_I16, QSSM_X_INT8, QSSM_X_SOFTEDGE, qssm_calib_block_absmax,
               qssm_calib_channel_absmax, qssm_calib_cluster_channels, qssm_calib_group_absmax,
               qssm_calib_s4d_state_scale, qssm_calib_scales, qssm_calib_softedge,
               qssm_softedge_track, qssm_softedge_track_workspace_size,
               qssm_quant_group_x, qssm_quant_state_group_BC, qssm_s4d_scan, qssm_scan_w8a8,
               qssm_scan_workspace_size, qssm_softedge_encode, qssm_ssd_chunk_int8,
               qssm_ssd_workspace_size, qssm_state_update, s4d_args, scan_args, ssd_args,
               update_args, gemm_args, qssm_gemm_w4a8, qssm_quant_w4)


def _dev(a, device, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


# ------------------------------------------------------------------------------------------------
# Calibration (host, offline)

def calib_x_groups(x_cal, G):
    """Quamba2 steps 1-2 on a calibration tensor [outer, C, inner]: per-channel absmax, sort and
    cluster into G groups, one scale per group. Returns (perm, group_of, scales)."""
    ch = qssm_calib_channel_absmax(x_cal)
    perm, group_of = qssm_calib_cluster_channels(ch, G)
    return perm, group_of, qssm_calib_scales(qssm_calib_group_absmax(ch[perm], group_of, G))


def calib_state_groups(bc_cal, gs):
    """Per-(group, state group) scales of B or C from a calibration tensor [outer, Gbc, N, inner]."""
    outer, Gbc, N, inner = bc_cal.shape
    ch = qssm_calib_channel_absmax(np.ascontiguousarray(bc_cal).reshape(outer, Gbc * N, inner))
    return qssm_calib_scales(qssm_calib_block_absmax(ch, gs))


def calib_y_groups(y_cal, G):
    """Static scales of a layer's int8 output from a calibration output [outer, C, inner]: the
    channels are clustered by absmax as x's are (Quamba2 steps 1-2) but stay in place, so the
    result is the group of each channel in its own order, and one scale per group."""
    ch = qssm_calib_channel_absmax(y_cal)
    perm, grp = qssm_calib_cluster_channels(ch, G)
    group_of = np.empty(ch.size, np.uint8)
    group_of[perm] = grp
    return group_of, qssm_calib_scales(qssm_calib_group_absmax(ch, group_of, G))


def calib_softedge(x_cal, perm, group_of, G, with_state=False):
    """Per-group soft-edge (s, L, H) from the calibration tensor in cluster order; with_state:
    also the fp64 EMA state [G, 2] an on-device tracker continues from."""
    xs = np.asarray(x_cal)[:, perm, :]
    s = np.zeros(G, np.float32)
    L = np.zeros(G, np.float32)
    H = np.zeros(G, np.float32)
    st = np.zeros((G, 2), np.float64)
    for g in range(G):
        s[g], L[g], H[g], st[g] = qssm_calib_softedge(xs[:, group_of == g, :])
    return (s, L, H, st) if with_state else (s, L, H)


def state_group_map(Gbc, N, gs):
    """Scale index of each of the Gbc * N states of B or C: g * (N / gs) + n / gs."""
    n = np.arange(Gbc * N)
    return ((n // N) * (N // gs) + (n % N) // gs).astype(np.uint8)


def calib_softedge_state_groups(bc_cal, gs):
    """Per-state-group soft-edge (s, L, H) of B or C [outer, Gbc, N, inner]."""
    bc = np.asarray(bc_cal)
    o, Gbc, N, inner = bc.shape
    return calib_softedge(bc.reshape(o, Gbc * N, inner), np.arange(Gbc * N),
                          state_group_map(Gbc, N, gs), Gbc * N // gs)


# ------------------------------------------------------------------------------------------------
# Mamba1 selective scan layer

class Mamba1Layer:
    """x, delta [B, D, L]; A [D, N]; B, C [B, Gbc, N, L]. One step = quantize x (gathered into
    cluster order), quantize B and C, run the W8A8 scan."""

    def __init__(self, inp, G, gs, device, x_code=QSSM_X_INT8, dynamic_scales=False,
                 y_dtype=QSSM_F32, with_h0=False, perm=True, y_out=None, bc_code=QSSM_X_INT8,
                 track=False, time_blocks=0):
        """y_out = (group_of [D] uint8, scales [Gy] fp32, bias [D] fp32 or None), in the layer's
        channel order: the scan then writes int8 y codes for the next W8A8 module.
        x_code / bc_code: int8 or a soft-edge form (QSSM_X_SOFTEDGE, QSSM_X_SOFTEDGE2) for x and
        for B/C (soft-edge B/C: per-state-group base scales and thresholds from the calibration
        draws). track (soft-edge x): every step first updates the x thresholds on the device from
        the step's own x (P5 / P99.9 with the EMA, continuing the calibration's state)."""
        import torch
        self.inp = inp
        self.G, self.gs, self.x_code = G, gs, x_code
        self.dynamic = dynamic_scales
        x = inp["x"]
        B, D, L = x.shape
        Gbc, N = inp["B"].shape[1], inp["B"].shape[2]
        if Gbc > 1 and not (dynamic_scales and not perm):
            # the cluster permutation is over all channels; with several B/C groups it would move
            # channels out of their group
            raise ValueError("several B/C groups need channels in their original order "
                             "(dynamic_scales=True, perm=False)")
        self.shape = (B, D, L, N, Gbc)
        if dynamic_scales:
            self.perm = np.arange(D, dtype=np.int32)
            self.group_of = np.zeros(D, np.uint8) if G == 1 else (np.arange(D) * G // D).astype(np.uint8)
            xs = np.ones(G, np.float32)
            bs = np.ones(Gbc * N // gs, np.float32)
            cs = np.ones(Gbc * N // gs, np.float32)
        else:
            self.perm, self.group_of, xs = calib_x_groups(inp["x_cal"], G)
            bs = calib_state_groups(inp["B_cal"], gs)
            cs = calib_state_groups(inp["C_cal"], gs)
        self.bc_code, self.track = bc_code, track
        if track and x_code == QSSM_X_INT8:
            raise ValueError("threshold tracking needs soft-edge x")
        if x_code != QSSM_X_INT8:
            xs, sL, sH, st = calib_softedge(inp["x_cal"], self.perm, self.group_of, G, with_state=True)
            self.sL, self.sH = _dev(sL, device), _dev(sH, device)
            self.ema = _dev(st, device)
            if track:
                self.track_ws = torch.empty(qssm_softedge_track_workspace_size(G), dtype=torch.uint8,
                                            device=device)
        if bc_code != QSSM_X_INT8:
            self.sg_map = _dev(state_group_map(Gbc, N, gs), device)
            bs, bL, bH = calib_softedge_state_groups(inp["B_cal"], gs)
            cs, cL, cH = calib_softedge_state_groups(inp["C_cal"], gs)
            self.bL, self.bH, self.cL, self.cH = (_dev(a, device) for a in (bL, bH, cL, cH))
        p = self.perm
        dev = device
        self.x = _dev(x, dev)
        self.Bf = _dev(inp["B"], dev)
        self.Cf = _dev(inp["C"], dev)
        self.delta = _dev(inp["delta"][:, p, :], dev)
        self.A = _dev(inp["A"][p], dev)
        self.D = _dev(inp["D"][p], dev)
        self.h0 = _dev(inp["h0"][:, p, :], dev) if with_h0 else None
        self.perm_t = None if (dynamic_scales and not perm) else _dev(p, dev)
        self.group_t = _dev(self.group_of, dev)
        self.xs = _dev(xs, dev)
        self.bs = _dev(bs, dev)
        self.cs = _dev(cs, dev)
        self.xq = torch.empty((B, D, L), dtype=torch.int8 if x_code == QSSM_X_INT8 else torch.uint8,
                              device=dev)
        bdt = torch.int8 if bc_code == QSSM_X_INT8 else torch.uint8
        self.Bq = torch.empty(inp["B"].shape, dtype=bdt, device=dev)
        self.Cq = torch.empty(inp["C"].shape, dtype=bdt, device=dev)
        ydt = torch.float32 if y_dtype == QSSM_F32 else torch.float16
        self.y_out = None
        if y_out is not None:
            ydt = torch.int8
            yg, ys, yb = y_out
            self.y_out = (_dev(np.asarray(yg, np.uint8), dev), _dev(np.asarray(ys, np.float32), dev),
                          None if yb is None else _dev(np.asarray(yb, np.float32), dev))
        self.y = torch.empty((B, D, L), dtype=ydt, device=dev)
        self.h_last = torch.empty((B, D, N), dtype=torch.float32, device=dev)
        yo = self.y_out or (None, None, None)
        self.args = scan_args(self.xq, x_code, self.group_t, self.xs, self.delta, self.A, self.Bq,
                              self.Cq, self.bs, self.cs, gs, self.y, Dskip=self.D, h0=self.h0,
                              h_last=self.h_last, y_group_of=yo[0], y_scales=yo[1], y_bias=yo[2],
                              bc_code=bc_code, time_blocks=time_blocks)
        self.ws = torch.empty(qssm_scan_workspace_size(self.args), dtype=torch.uint8, device=dev)

    def quantize(self):
        x3 = self.x
        if self.x_code == QSSM_X_INT8:
            qssm_quant_group_x(x3, self.group_t, self.G, self.xs, self.xq, perm=self.perm_t,
                               compute_scales=self.dynamic)
        else:
            if self.track:
                qssm_softedge_track(x3, self.group_t, self.G, self.ema, self.xs, self.sL, self.sH,
                                    self.track_ws, ema_valid=True, perm=self.perm_t)
            qssm_softedge_encode(x3, self.group_t, self.G, self.xs, self.sL, self.sH, self.xq,
                                 perm=self.perm_t, form=self.x_code)
        if self.bc_code == QSSM_X_INT8:
            qssm_quant_state_group_BC(self.Bf, self.gs, self.bs, self.Bq,
                                      compute_scales=self.dynamic)
            qssm_quant_state_group_BC(self.Cf, self.gs, self.cs, self.Cq,
                                      compute_scales=self.dynamic)
        else:
            B, Gbc, N, L = self.Bf.shape
            ng = Gbc * N // self.gs
            for src, dst, sc, lo, hi in ((self.Bf, self.Bq, self.bs, self.bL, self.bH),
                                         (self.Cf, self.Cq, self.cs, self.cL, self.cH)):
                qssm_softedge_encode(src.view(B, Gbc * N, L), self.sg_map, ng, sc, lo, hi,
                                     dst.view(B, Gbc * N, L), form=self.bc_code)

    def scan(self):
        qssm_scan_w8a8(self.args, self.ws)

    def step(self):
        self.quantize()
        self.scan()
        return self.y


# ------------------------------------------------------------------------------------------------
# S4D layer

class S4dLayer:
    """Pixel sequence u [B, L] lifted by int8 weights w [H]; int8 A, B, C planes with per-channel
    (Re and Im separate) scales; fp32 or int16 state. One step = quantize u, run the scan (the
    parameter codes are static, quantized once at set-up with the same library quantizer)."""

    PLANES = ("A_re", "A_im", "B_re", "B_im", "C_re", "C_im")

    def __init__(self, inp, device, state_dtype=QSSM_F32, state_scale=None, with_h0=False):
        import torch
        dev = device
        self.inp = inp
        u = inp["u"]
        B, L = u.shape
        H, N = inp["A_re"].shape
        self.shape = (B, L, H, N)
        ident = np.arange(H, dtype=np.uint8) if H <= 256 else None
        # per-tensor scale for the input and the lift weights, per-channel for the planes
        self.u_f = _dev(u.reshape(B, 1, L), dev)
        self.u_scale = _dev(qssm_calib_scales(qssm_calib_channel_absmax(u.reshape(1, 1, -1))), dev)
        self.uq = torch.empty((B, 1, L), dtype=torch.int8, device=dev)
        self.w_scale = _dev(qssm_calib_scales(qssm_calib_channel_absmax(inp["w"].reshape(1, 1, -1))), dev)
        self.wq = torch.empty((1, 1, H), dtype=torch.int8, device=dev)
        qssm_quant_group_x(_dev(inp["w"].reshape(1, 1, H), dev), _dev(np.zeros(1, np.uint8), dev), 1,
                           self.w_scale, self.wq)
        self.params, self.scales = {}, {}
        assert ident is not None, "per-channel plane scales need H <= 256"
        gid = _dev(ident, dev)
        for k in self.PLANES:
            v = inp[k].reshape(1, H, N)
            sc = qssm_calib_scales(qssm_calib_channel_absmax(v))
            self.scales[k] = _dev(sc, dev)
            self.params[k] = torch.empty((H, N), dtype=torch.int8, device=dev)
            qssm_quant_group_x(_dev(v, dev), gid, H, self.scales[k], self.params[k].view(1, H, N))
        self.log_dt = _dev(inp["log_dt"], dev)
        self.D = _dev(inp["D"], dev)
        self.state_dtype = state_dtype
        if state_dtype == QSSM_I16 and state_scale is None:
            # int16 state without a given scale: the library's bound from the quantized parameters
            # (|u| <= u_scale * w_scale * 128 * |w code| per channel, headroom 1.25)
            host = {k: self.params[k].cpu().numpy() for k in ("A_re", "B_re", "B_im")}
            hs = {k: self.scales[k].cpu().numpy() for k in ("A_re", "B_re", "B_im")}
            wq = self.wq.cpu().numpy().reshape(-1).astype(np.float32)
            umax = (self.u_scale.cpu().numpy()[0] * self.w_scale.cpu().numpy()[0] * np.float32(128.0)
                    * np.abs(wq)).astype(np.float32)
            state_scale = qssm_calib_s4d_state_scale(L, host["A_re"], hs["A_re"], host["B_re"],
                                                     hs["B_re"], host["B_im"], hs["B_im"],
                                                     inp["log_dt"], umax)
        self.state_scale_host = None if state_scale is None else np.asarray(state_scale, np.float32)
        self.state_scale = None if state_scale is None else _dev(self.state_scale_host, dev)
        sdt = torch.float32 if state_dtype == QSSM_F32 else torch.int16
        self.h0 = None
        if with_h0:
            h0 = np.stack([inp["h0_re"], inp["h0_im"]], axis=-1)
            if state_dtype == QSSM_I16:
                s64 = np.asarray(state_scale, np.float32).astype(np.float64)[None, :, None, None]
                h0 = np.clip(np.rint(h0.astype(np.float64) / s64), -32768, 32767)
            self.h0 = _dev(h0, dev, sdt)
        self.y = torch.empty((B, H, L), dtype=torch.float32, device=dev)
        self.h_last = torch.empty((B, H, N, 2), dtype=sdt, device=dev)
        self.args = s4d_args(self.uq, self.u_scale, self.params, self.scales, self.log_dt, self.y,
                             wq=self.wq.view(H), w_scale=self.w_scale, Dskip=self.D,
                             state_dtype=state_dtype, state_scale=self.state_scale, h0=self.h0,
                             h_last=self.h_last)

    def step(self):
        qssm_quant_group_x(self.u_f, _ZERO_GROUP(self.u_f.device), 1, self.u_scale, self.uq)
        qssm_s4d_scan(self.args)
        return self.y


_zero_cache = {}


def _ZERO_GROUP(device):
    import torch
    key = str(device)
    if key not in _zero_cache:
        _zero_cache[key] = torch.zeros(1, dtype=torch.uint8, device=device)
    return _zero_cache[key]


# ------------------------------------------------------------------------------------------------
# Mamba2 SSD layer

def calib_ssd_x_groups(x_cal, nheads, headdim, ngroups, groups_per_block):
    """x channels (h, p) clustered within each head block (the heads sharing one B/C group) into
    groups_per_block groups; returns group_of [nh * P] and scales [ngroups * groups_per_block]."""
    C = nheads * headdim
    xc = np.ascontiguousarray(x_cal).reshape(-1, C, 1)
    ch = qssm_calib_channel_absmax(xc)
    per_block = C // ngroups
    group_of = np.empty(C, np.uint8)
    for k in range(ngroups):
        sl = slice(k * per_block, (k + 1) * per_block)
        perm, grp = qssm_calib_cluster_channels(ch[sl], groups_per_block)
        blk = np.empty(per_block, np.uint8)
        blk[perm] = grp + np.uint8(k * groups_per_block)
        group_of[sl] = blk
    return group_of, qssm_calib_scales(qssm_calib_group_absmax(ch, group_of,
                                                               ngroups * groups_per_block))


class SsdLayer:
    """x [B, L, nh, P], delta [B, L, nh], B/C [B, L, Gbc, N]. One step = quantize x, B, C, run the
    chunked SSD."""

    def __init__(self, inp, device, chunk=256, gs=16, groups_per_block=8, y_dtype=QSSM_F32,
                 with_h0=False, state_mma=0, y_out=None, intra_mma=0):
        """y_out = (group_of [nh * P] uint8, scales [Gy] fp32, bias [nh * P] fp32 or None): the
        layer then writes int8 y codes for the next W8A8 module. state_mma / intra_mma select
        int8 MFMA (QSSM_MMA_I8) for the chunk state / the intra-chunk product."""
        import torch
        dev = device
        x = inp["x"]
        B, L, nh, P = x.shape
        Gbc, N = inp["B"].shape[2], inp["B"].shape[3]
        self.shape = (B, L, nh, P, N, Gbc)
        self.gs, self.chunk = gs, chunk
        self.group_of, xs = calib_ssd_x_groups(inp["x_cal"], nh, P, Gbc, groups_per_block)
        bs = calib_state_groups(np.moveaxis(inp["B_cal"], 1, -1), gs)
        cs = calib_state_groups(np.moveaxis(inp["C_cal"], 1, -1), gs)
        self.G = xs.size
        self.x = _dev(x, dev)
        self.Bf = _dev(inp["B"], dev)
        self.Cf = _dev(inp["C"], dev)
        self.delta = _dev(inp["delta"], dev)
        self.A = _dev(inp["A"], dev)
        self.D = _dev(inp["D"], dev)
        self.h0 = _dev(inp["h0"], dev) if with_h0 else None
        self.group_t = _dev(self.group_of, dev)
        self.xs, self.bs, self.cs = _dev(xs, dev), _dev(bs, dev), _dev(cs, dev)
        self.xq = torch.empty(x.shape, dtype=torch.int8, device=dev)
        self.Bq = torch.empty(inp["B"].shape, dtype=torch.int8, device=dev)
        self.Cq = torch.empty(inp["C"].shape, dtype=torch.int8, device=dev)
        ydt = torch.float32 if y_dtype == QSSM_F32 else torch.float16
        yo = (None, None, None)
        if y_out is not None:
            ydt = torch.int8
            yg, ys, yb = y_out
            yo = (_dev(np.asarray(yg, np.uint8), dev), _dev(np.asarray(ys, np.float32), dev),
                  None if yb is None else _dev(np.asarray(yb, np.float32), dev))
        self.y_out = yo
        self.y = torch.empty(x.shape, dtype=ydt, device=dev)
        self.h_last = torch.empty((B, nh, P, N), dtype=torch.float32, device=dev)
        self.args = ssd_args(self.xq, self.group_t, self.xs, self.delta, self.A, self.Bq, self.Cq,
                             self.bs, self.cs, gs, chunk, self.y, Dskip=self.D, h0=self.h0,
                             h_last=self.h_last, state_mma=state_mma, intra_mma=intra_mma,
                             y_group_of=yo[0],
                             y_scales=yo[1], y_bias=yo[2])
        self.ws = torch.empty(max(qssm_ssd_workspace_size(self.args), 1), dtype=torch.uint8,
                              device=dev)

    def quantize(self):
        B, L, nh, P, N, Gbc = self.shape
        qssm_quant_group_x(self.x.view(B * L, nh * P, 1), self.group_t, self.G, self.xs,
                           self.xq.view(B * L, nh * P, 1))
        qssm_quant_state_group_BC(self.Bf.view(B * L, Gbc, N, 1), self.gs, self.bs,
                                  self.Bq.view(B * L, Gbc, N, 1))
        qssm_quant_state_group_BC(self.Cf.view(B * L, Gbc, N, 1), self.gs, self.cs,
                                  self.Cq.view(B * L, Gbc, N, 1))

    def scan(self):
        qssm_ssd_chunk_int8(self.args, self.ws)

    def step(self):
        self.quantize()
        self.scan()
        return self.y


# ------------------------------------------------------------------------------------------------
# Decode

class DecodeLayer:
    """Static scales from one calibration step; state [B, nh, P, N] fp32 or fp16, updated in place.
    One step = one fused state-update call for a new token of every sequence."""

    def __init__(self, params, device, gs=16, groups_per_block=8, state_dtype=QSSM_F32,
                 emit_codes=False, y_out=None):
        """y_out = (group_of [nh * P] uint8, scales [Gy] fp32, bias [nh * P] fp32 or None): int8
        y codes for the next W8A8 module."""
        import torch
        dev = device
        st0 = params["state0"]
        B, nh, P, N = st0.shape
        Gbc = params["B_cal"].shape[1]
        self.shape = (B, nh, P, N, Gbc)
        self.gs = gs
        self.group_of, xs = calib_ssd_x_groups(params["x_cal"].reshape(B, nh * P), nh, P, Gbc,
                                               groups_per_block)
        bs = calib_state_groups(params["B_cal"][..., None], gs)
        cs = calib_state_groups(params["C_cal"][..., None], gs)
        self.group_t = _dev(self.group_of, dev)
        self.xs, self.bs, self.cs = _dev(xs, dev), _dev(bs, dev), _dev(cs, dev)
        self.A = _dev(params["A"], dev)
        self.D = _dev(params["D"], dev)
        sdt = torch.float32 if state_dtype == QSSM_F32 else torch.float16
        self.state = _dev(st0, dev, sdt)
        yo = (None, None, None)
        if y_out is not None:
            yg, ys, yb = y_out
            yo = (_dev(np.asarray(yg, np.uint8), dev), _dev(np.asarray(ys, np.float32), dev),
                  None if yb is None else _dev(np.asarray(yb, np.float32), dev))
        self.y_out = yo
        self.y = torch.empty((B, nh, P), dtype=torch.float32 if y_out is None else torch.int8,
                             device=dev)
        self.x = torch.empty((B, nh, P), dtype=torch.float32, device=dev)
        self.Bm = torch.empty((B, Gbc, N), dtype=torch.float32, device=dev)
        self.Cm = torch.empty((B, Gbc, N), dtype=torch.float32, device=dev)
        self.delta = torch.empty((B, nh), dtype=torch.float32, device=dev)
        self.codes = None
        if emit_codes:
            self.codes = (torch.empty((B, nh, P), dtype=torch.int8, device=dev),
                          torch.empty((B, Gbc, N), dtype=torch.int8, device=dev),
                          torch.empty((B, Gbc, N), dtype=torch.int8, device=dev))
        c = self.codes or (None, None, None)
        self.args = update_args(self.x, self.group_t, self.xs, self.Bm, self.Cm, self.bs, self.cs, gs,
                                self.delta, self.A, self.state, self.y, Dskip=self.D, xq_out=c[0],
                                Bq_out=c[1], Cq_out=c[2], y_group_of=yo[0], y_scales=yo[1],
                                y_bias=yo[2])

    def load_inputs(self, step_inputs):
        """Copies one step's host inputs into the resident device buffers (outside timed regions)."""
        import torch
        for name, buf in (("x", self.x), ("B", self.Bm), ("C", self.Cm), ("delta", self.delta)):
            buf.copy_(torch.from_numpy(np.ascontiguousarray(step_inputs[name])))

    def step(self):
        qssm_state_update(self.args)
        return self.y


# ------------------------------------------------------------------------------------------------
# W4A8 linear layer

class W4A8Linear:
    """y = x W^T (+ bias) with 4-bit weights [N, K] quantized offline (per output channel and
    group of input channels) and int8 activations with one static scale. One step = quantize the
    fp32 activations [M, K] to int8, then the W4A8 GEMM."""

    def __init__(self, w, x, x_cal, device, group=None, bias=None, y_dtype=QSSM_F32):
        import torch
        dev = device
        N, K = w.shape
        M = x.shape[0]
        self.group = K if group is None else group
        self.shape = (M, N, K)
        ws, wp = qssm_quant_w4(w, self.group)
        self.w_scales_host, self.w_packed_host = ws, wp
        self.xs = _dev(qssm_calib_scales(qssm_calib_channel_absmax(
            np.ascontiguousarray(x_cal, np.float32).reshape(1, 1, -1))), dev)
        self.x = _dev(np.ascontiguousarray(x, np.float32), dev)
        self.xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        self.w = _dev(wp, dev)
        self.ws = _dev(ws, dev)
        self.bias = None if bias is None else _dev(np.asarray(bias, np.float32), dev)
        self.y = torch.empty((M, N), dtype=torch.float32 if y_dtype == QSSM_F32 else torch.float16,
                             device=dev)
        self.zero_group = torch.zeros(1, dtype=torch.uint8, device=dev)
        self.args = gemm_args(self.xq, self.xs, self.w, self.ws, self.group, self.y, bias=self.bias)

    def quantize(self):
        M, N, K = self.shape
        qssm_quant_group_x(self.x.view(1, 1, M * K), self.zero_group, 1, self.xs,
                           self.xq.view(1, 1, M * K))

    def gemm(self):
        qssm_gemm_w4a8(self.args)

    def step(self):
        self.quantize()
        self.gemm()
        return self.y
