"""Whole-workload oracle paths — TEST INFRASTRUCTURE ONLY.

Each function takes the seeded fp32 inputs of ``qssm_synth`` and runs the method with the oracle's
own pieces only: offline calibration (Quamba2 steps 1-3, Quamba-SE 4.1), quantization to codes,
exact fp64 dequantization, and the fp64 recurrence. Nothing here calls the HIP library.
"""
from __future__ import annotations

import numpy as np

from . import (cluster_channels, decode_step, dequant_group, dequant_state_group, finite_absmax,
               group_scales, quant_group_x, quant_state_group, s4d_scan, scale_from_absmax,
               selective_scan, softedge_encode, softedge_thresholds, softedge_track,
               softedge_values, ssd_chunked, ssd_as_sequential, state_group_scales)


# ------------------------------------------------------------------------------------------------
# calibration

def calib_x(x_cal, G):
    """Sort/cluster channels of x_cal [outer, C, inner] into G groups; returns (perm, group_of,
    scales) with scales from the group absmax of the calibration tensor."""
    ch = finite_absmax(x_cal, axis=(0, 2))
    perm, group_of = cluster_channels(ch, G)
    g_abs = np.zeros(G, np.float32)
    for c in range(ch.size):
        g = group_of[c]
        g_abs[g] = max(g_abs[g], ch[perm[c]])
    return perm, group_of, scale_from_absmax(g_abs)


def calib_softedge(x_cal, perm, group_of, G, with_state=False):
    """Per-group soft-edge (s, L, H) as a [3, G] array; with_state: also the fp64 (L, H) pairs
    an EMA continues from."""
    xs = np.asarray(x_cal)[:, perm, :]
    out = np.zeros((3, G), np.float32)
    states = []
    for g in range(G):
        s, L, H, st = softedge_thresholds(xs[:, group_of == g, :])
        out[:, g] = (s, L, H)
        states.append(st)
    return (out, states) if with_state else out


def state_group_map(Gbc, N, gs):
    """Scale index of each of the Gbc * N states (B/C group g, state n): g * (N / gs) + n / gs."""
    n = np.arange(Gbc * N)
    return ((n // N) * (N // gs) + (n % N) // gs).astype(np.uint8)


def calib_softedge_state_groups(bc_cal, gs):
    """Soft-edge (s, L, H) [3, Gbc * N / gs] of B or C [outer, Gbc, N, inner], one per state group."""
    bc = np.asarray(bc_cal)
    o, Gbc, N, inner = bc.shape
    return calib_softedge(bc.reshape(o, Gbc * N, inner), np.arange(Gbc * N),
                          state_group_map(Gbc, N, gs), Gbc * N // gs)


def calib_ssd_x(x_cal, nheads, headdim, ngroups, groups_per_block):
    """Clustering within each head block (heads sharing a B/C group)."""
    C = nheads * headdim
    ch = finite_absmax(np.asarray(x_cal).reshape(-1, C), axis=0)
    per_block = C // ngroups
    group_of = np.empty(C, np.uint8)
    g_abs = np.zeros(ngroups * groups_per_block, np.float32)
    for k in range(ngroups):
        blk = ch[k * per_block:(k + 1) * per_block]
        perm, grp = cluster_channels(blk, groups_per_block)
        for pos in range(per_block):
            c = int(perm[pos])
            gid = k * groups_per_block + int(grp[pos])
            group_of[k * per_block + c] = gid
            g_abs[gid] = max(g_abs[gid], blk[c])
    return group_of, scale_from_absmax(g_abs)


# ------------------------------------------------------------------------------------------------
# Mamba1

def mamba1_calib(inp, G, gs, soft_edge=False, bc_soft_edge=False):
    """Offline calibration of the Mamba1 layer from its calibration draws."""
    perm, group_of, xs = calib_x(inp["x_cal"], G)
    c = dict(perm=perm, group_of=group_of, xs=xs, bs=state_group_scales(inp["B_cal"], gs),
             cs=state_group_scales(inp["C_cal"], gs))
    if soft_edge:
        c["se"], c["se_state"] = calib_softedge(inp["x_cal"], perm, group_of, G, with_state=True)
    if bc_soft_edge:
        c["bse"] = calib_softedge_state_groups(inp["B_cal"], gs)
        c["cse"] = calib_softedge_state_groups(inp["C_cal"], gs)
    return c


def _bc_softedge(bc, gs, se, ratio):
    """Soft-edge bytes of B or C [outer, Gbc, N, inner] with per-state-group (s, L, H), and their
    exact values."""
    o, Gbc, N, inner = bc.shape
    sg = state_group_map(Gbc, N, gs)
    q = softedge_encode(np.asarray(bc, np.float32).reshape(o, Gbc * N, inner), sg, se[0], se[1],
                        se[2], ratio=ratio)
    v = softedge_values(q, sg, se[0], ratio=ratio)
    return q.reshape(bc.shape), v.reshape(bc.shape)


def mamba1(inp, G, gs, soft_edge=False, dynamic=False, rows=None, with_h0=False, calib=None,
           se_ratio=4, bc_soft_edge=0, track=False):
    """Returns dict with perm, group_of, x/B/C scales, codes, and (for the selected (b, d) rows,
    all when rows is None) y and h_last in fp64. rows = (b_index_array, d_index_array).
    calib: a precomputed mamba1_calib result (static scales).
    soft_edge: x in soft-edge bytes with mode ratio se_ratio (4, or 2 for the shift-only form).
    track: the x thresholds of this batch come from the section 4.1 EMA update, continuing the
    calibration's state with this batch's own percentiles (softedge_track).
    bc_soft_edge: 0 for int8 B/C, else the mode ratio of soft-edge B/C bytes (per-state-group base
    scales and thresholds from the calibration draws)."""
    x = inp["x"]
    B, D, L = x.shape
    if calib is not None:
        perm, group_of, xs, bs, cs = (calib[k] for k in ("perm", "group_of", "xs", "bs", "cs"))
    elif dynamic:
        perm = np.arange(D, dtype=np.int32)
        group_of = np.zeros(D, np.uint8) if G == 1 else (np.arange(D) * G // D).astype(np.uint8)
        xs = group_scales(x, group_of, G, perm)
        bs = state_group_scales(inp["B"], gs)
        cs = state_group_scales(inp["C"], gs)
    else:
        perm, group_of, xs = calib_x(inp["x_cal"], G)
        bs = state_group_scales(inp["B_cal"], gs)
        cs = state_group_scales(inp["C_cal"], gs)
    out = dict(perm=perm, group_of=group_of, bs=bs, cs=cs)
    if soft_edge:
        if calib is not None and "se" in calib:
            se, st = calib["se"], calib["se_state"]
        else:
            se, st = calib_softedge(inp["x_cal"], perm, group_of, G, with_state=True)
        s, Lt, Ht = se
        if track:
            s, Lt, Ht, st = softedge_track(x, group_of, G, perm=perm, prev=st)
        out.update(xs=s, L=Lt, H=Ht, se_state=st)
        xq = softedge_encode(x, group_of, s, Lt, Ht, perm=perm, ratio=se_ratio)
    else:
        out["xs"] = xs
        xq = quant_group_x(x, group_of, xs, perm=perm)
    if bc_soft_edge:
        bse = calib["bse"] if calib is not None and "bse" in calib else \
            calib_softedge_state_groups(inp["B_cal"], gs)
        cse = calib["cse"] if calib is not None and "cse" in calib else \
            calib_softedge_state_groups(inp["C_cal"], gs)
        Bq, Bv = _bc_softedge(inp["B"], gs, bse, bc_soft_edge)
        Cq, Cv = _bc_softedge(inp["C"], gs, cse, bc_soft_edge)
        out.update(bs=bse[0], cs=cse[0], bse=bse, cse=cse)
    else:
        Bq = quant_state_group(inp["B"], gs, bs)
        Cq = quant_state_group(inp["C"], gs, cs)
        Bv = Cv = None
    out.update(xq=xq, Bq=Bq, Cq=Cq)
    delta, A, Dk = inp["delta"][:, perm], inp["A"][perm], inp["D"][perm]
    h0 = inp["h0"][:, perm] if with_h0 else None
    bsel = np.arange(B) if rows is None else np.asarray(rows[0])
    dsel = np.arange(D) if rows is None else np.asarray(rows[1])
    ys, hs = [], []
    for b in np.unique(bsel):
        ds = dsel[bsel == b] if rows is not None else dsel
        xq_b = xq[b:b + 1][:, ds]
        if soft_edge:
            xh = softedge_values(xq_b, group_of[ds], out["xs"], ratio=se_ratio)
        else:
            xh = dequant_group(xq_b, group_of[ds], out["xs"])
        Bh = Bv[b:b + 1] if Bv is not None else dequant_state_group(Bq[b:b + 1], gs, bs)
        Ch = Cv[b:b + 1] if Cv is not None else dequant_state_group(Cq[b:b + 1], gs, cs)
        y, hl = selective_scan(xh, delta[b:b + 1][:, ds], A[ds], Bh, Ch, Dk[ds],
                               None if h0 is None else h0[b:b + 1][:, ds])
        ys.append(y[0])
        hs.append(hl[0])
    if rows is None:
        out["y"], out["h_last"] = np.stack(ys), np.stack(hs)
    else:
        out["y_rows"], out["h_rows"] = np.concatenate(ys), np.concatenate(hs)
    return out


# ------------------------------------------------------------------------------------------------
# S4D

PLANES = ("A_re", "A_im", "B_re", "B_im", "C_re", "C_im")


def s4d(inp, state_scale=None, with_h0=False):
    """Oracle S4D layer: per-tensor scales for the pixel input and the lift weights, per-channel
    (Re and Im separate) scales for the A, B, C planes; fp64 recurrence."""
    u = inp["u"]
    B, L = u.shape
    H, N = inp["A_re"].shape
    su = scale_from_absmax(finite_absmax(u, axis=(0, 1)))
    sw = scale_from_absmax(finite_absmax(inp["w"], axis=0))
    uq = quant_group_x(u.reshape(B, 1, L), np.zeros(1, np.uint8), [su])[:, 0, :]
    wq = quant_group_x(inp["w"].reshape(1, 1, H), np.zeros(1, np.uint8), [sw])[0, 0]
    codes, scales, deq = {}, {}, {}
    for k in PLANES:
        v = inp[k]
        sc = scale_from_absmax(finite_absmax(v, axis=1))
        q = quant_group_x(v.reshape(1, H, N), np.arange(H, dtype=np.uint8), sc)[0]
        codes[k], scales[k] = q, sc
        deq[k] = sc.astype(np.float64)[:, None] * q.astype(np.float64)
    Ah = deq["A_re"] + 1j * deq["A_im"]
    Bh = deq["B_re"] + 1j * deq["B_im"]
    Ch = deq["C_re"] + 1j * deq["C_im"]
    uh = (float(su) * float(sw)) * (uq.astype(np.float64)[:, None, :] * wq.astype(np.float64)[None, :, None])
    dt = np.exp(inp["log_dt"].astype(np.float64))
    h0 = None
    if with_h0:
        h0 = inp["h0_re"].astype(np.float64) + 1j * inp["h0_im"].astype(np.float64)
        if state_scale is not None:
            s = np.asarray(state_scale, np.float64)[None, :, None]
            h0 = s * np.clip(np.rint(h0.real / s), -32768, 32767) + \
                1j * s * np.clip(np.rint(h0.imag / s), -32768, 32767)
    y, hl = s4d_scan(uh, Ah, Bh, Ch, dt, Dskip=inp["D"],
                     state_scale=None if state_scale is None else np.asarray(state_scale, np.float64),
                     h0=h0)
    return dict(uq=uq, wq=wq, su=su, sw=sw, codes=codes, scales=scales, y=y, h_last=hl)


def s4d_state_scale(inp, headroom=1.25, with_h0=False):
    """Per-channel int16 state scale from the fp64 run: headroom * max |Re|, |Im| of the state over
    (b, t, n) / 32767 (the state sensitivity reading of the S4D page). A channel whose state never
    leaves 0 gets the smallest valid scale."""
    u = inp["u"]
    B, L = u.shape
    H, N = inp["A_re"].shape
    ref = s4d(inp)
    # rerun keeping every state: a short loop over t in fp64 is fine at this size
    from . import s4d_zoh
    su, sw = float(ref["su"]), float(ref["sw"])
    deq = {k: ref["scales"][k].astype(np.float64)[:, None] * ref["codes"][k] for k in PLANES}
    uh = su * sw * (ref["uq"].astype(np.float64)[:, None, :] * ref["wq"].astype(np.float64)[None, :, None])
    dt = np.exp(inp["log_dt"].astype(np.float64))
    m = np.zeros(H)
    for h in range(H):
        Ab, Bb = s4d_zoh(deq["A_re"][h] + 1j * deq["A_im"][h], deq["B_re"][h] + 1j * deq["B_im"][h], dt[h])
        st = np.zeros((B, N), np.complex128)
        if with_h0:
            st = inp["h0_re"][:, h].astype(np.float64) + 1j * inp["h0_im"][:, h].astype(np.float64)
            m[h] = max(np.abs(st.real).max(), np.abs(st.imag).max())
        for t in range(L):
            st = Ab[None, :] * st + Bb[None, :] * uh[:, h, t][:, None]
            m[h] = max(m[h], np.abs(st.real).max(), np.abs(st.imag).max())
    return np.maximum(headroom * m / 32767.0, 2.0 ** -100).astype(np.float32)


# ------------------------------------------------------------------------------------------------
# SSD

def ssd(inp, chunk=256, gs=16, groups_per_block=8, with_h0=False, heads=None, int8_state=False,
        exact=False, calib=None, int8_intra=False):
    """Oracle SSD layer. heads: optional subset of head indices (the recurrence of each head is
    independent; B/C groups follow the head). int8_state selects the requantized int8 chunk state,
    int8_intra the row-requantized int8 intra-chunk output; exact=True runs the plain sequential
    scan instead of the chunked form. calib: optional
    (group_of, xs, bs, cs) used instead of the calibration from inp (tests set scales outside the
    valid range this way). Returns codes, scales and fp64 y / h_last (for the selected heads:
    y [B, L, len(heads), P])."""
    x = inp["x"]
    B, L, nh, P = x.shape
    Gbc, N = inp["B"].shape[2], inp["B"].shape[3]
    if calib is None:
        group_of, xs = calib_ssd_x(inp["x_cal"], nh, P, Gbc, groups_per_block)
        bs = state_group_scales(np.moveaxis(inp["B_cal"], 1, -1), gs)
        cs = state_group_scales(np.moveaxis(inp["C_cal"], 1, -1), gs)
    else:
        group_of, xs, bs, cs = calib
    xq = quant_group_x(x.reshape(B * L, nh * P, 1), group_of, xs).reshape(x.shape)
    Bq = quant_state_group(inp["B"].reshape(B * L, Gbc, N, 1), gs, bs).reshape(inp["B"].shape)
    Cq = quant_state_group(inp["C"].reshape(B * L, Gbc, N, 1), gs, cs).reshape(inp["C"].shape)
    out = dict(group_of=group_of, xs=xs, bs=bs, cs=cs, xq=xq, Bq=Bq, Cq=Cq)
    hsel = np.arange(nh) if heads is None else np.asarray(heads)
    hpg = nh // Gbc
    sx = xs.astype(np.float64)[group_of].reshape(nh, P)
    ys, hls = [], []
    for h in hsel:
        g = h // hpg
        xh = xq[:, :, h:h + 1, :].astype(np.float64) * sx[h][None, None, None, :]
        Bh = dequant_state_group(np.moveaxis(Bq[:, :, g:g + 1, :], 1, -1), gs,
                                 bs.reshape(Gbc, -1)[g]).transpose(0, 3, 1, 2)
        Ch = dequant_state_group(np.moveaxis(Cq[:, :, g:g + 1, :], 1, -1), gs,
                                 cs.reshape(Gbc, -1)[g]).transpose(0, 3, 1, 2)
        h0 = inp["h0"][:, h:h + 1] if with_h0 else None
        args = (xh, inp["delta"][:, :, h:h + 1], inp["A"][h:h + 1], Bh, Ch)
        if exact:
            y, hl = ssd_as_sequential(*args, Dskip=inp["D"][h:h + 1], h0=h0)
        else:
            y, hl = ssd_chunked(*args, chunk, Dskip=inp["D"][h:h + 1], h0=h0,
                                int8_state=int8_state, qx=xq[:, :, h:h + 1, :], sx=sx[h],
                                int8_intra=int8_intra)
        ys.append(y[:, :, 0])
        hls.append(hl[:, 0])
        if int8_intra:
            out.setdefault("intra_w", []).append((h, Bh[:, :, 0], Ch[:, :, 0], xh[:, :, 0]))
    out["y"] = np.stack(ys, axis=2)
    out["h_last"] = np.stack(hls, axis=1)
    return out


def ssd_intra_near_boundary(inp, ref, eps_rel, eps_abs, chunk=256):
    """For a run of ssd(..., int8_intra=True): per output [B, L, len(heads), P], the sum over the
    row's requantized weights whose scaled value t = W * 127 / m_i lies within
    eps_rel |t| + eps_abs of a rounding boundary of (m_i / 127) |xh_j[p]|: how far a computation
    of W carrying relative error eps_rel can move that output by deciding those codes the other
    way. W, m_i and xh are the oracle's own (fp64, from the dequantized codes). Also returns the
    number of such codes and of all codes."""
    B, L = inp["x"].shape[:2]
    P = inp["x"].shape[3]
    out = np.zeros((B, L, len(ref["intra_w"]), P))
    near_total = codes_total = 0
    for k, (h, Bh, Ch, xh) in enumerate(ref["intra_w"]):
        for b in range(B):
            for t0 in range(0, L, chunk):
                q = min(chunk, L - t0)
                dt = np.asarray(inp["delta"][b, t0:t0 + q, h], np.float64)
                cum = np.cumsum(dt * np.float64(inp["A"][h]))
                CB = Ch[b, t0:t0 + q] @ Bh[b, t0:t0 + q].T
                W = np.tril(CB * np.exp(cum[:, None] - cum[None, :]) * dt[None, :])
                m = np.abs(W).max(axis=1)
                with np.errstate(divide="ignore", invalid="ignore"):
                    t = np.where(m[:, None] > 0, W * 127 / m[:, None], 0.0)
                near = np.abs(t - np.floor(t) - 0.5) < eps_rel * np.abs(t) + eps_abs
                near &= np.tri(q, dtype=bool)
                near_total += int(near.sum())
                codes_total += q * (q + 1) // 2
                out[b, t0:t0 + q, k, :] = (m / 127)[:, None] * (near @ np.abs(xh[b, t0:t0 + q]))
    return out, near_total, codes_total


# ------------------------------------------------------------------------------------------------
# Decode

def decode(params, step_inputs, gs=16, groups_per_block=8, batches=None):
    """Runs len(step_inputs) decode steps in fp64 from params['state0']. batches: optional subset of
    sequences (each sequence's state is independent). Returns codes and y per step and the final
    state."""
    st0 = params["state0"]
    B, nh, P, N = st0.shape
    Gbc = params["B_cal"].shape[1]
    group_of, xs = calib_ssd_x(params["x_cal"].reshape(B, nh * P), nh, P, Gbc, groups_per_block)
    bs = state_group_scales(params["B_cal"][..., None], gs)
    cs = state_group_scales(params["C_cal"][..., None], gs)
    bsel = np.arange(B) if batches is None else np.asarray(batches)
    state = st0[bsel].astype(np.float64).copy()
    sx = xs.astype(np.float64)[group_of].reshape(nh, P)
    res = dict(group_of=group_of, xs=xs, bs=bs, cs=cs, xq=[], Bq=[], Cq=[], y=[])
    for inp in step_inputs:
        x, Bm, Cm, dl = inp["x"][bsel], inp["B"][bsel], inp["C"][bsel], inp["delta"][bsel]
        nb = len(bsel)
        xq = quant_group_x(x.reshape(nb, nh * P, 1), group_of, xs).reshape(nb, nh, P)
        Bq = quant_state_group(Bm[..., None], gs, bs)[..., 0]
        Cq = quant_state_group(Cm[..., None], gs, cs)[..., 0]
        xh = xq.astype(np.float64) * sx[None]
        Bh = dequant_state_group(Bq[..., None], gs, bs)[..., 0]
        Ch = dequant_state_group(Cq[..., None], gs, cs)[..., 0]
        y = decode_step(xh, Bh, Ch, dl, params["A"], state, Dskip=params["D"])
        for k, v in (("xq", xq), ("Bq", Bq), ("Cq", Cq), ("y", y)):
            res[k].append(v)
    res["state"] = state
    return res
