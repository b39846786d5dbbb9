"""Seeded synthetic inputs for the quantized state-space hot path.

This module only draws random tensors (numpy ``default_rng([config, stream])``). It holds none of
the method's arithmetic: no quantization, no scales, no clustering, no recurrence. Both the HIP
library's tests/benchmarks and the oracle consume the same draws.

The shapes and distributions stand in for the pages' workloads, which are not available here:
  tiny Mamba1 layer                      (c1)
  S4D on sequential-MNIST-shaped input   (c2: 784 = 28*28 pixel steps; the dataset is absent)
  Mamba1-130M-shaped layer activations   (c3: Student-t x with rare x100 outliers)
  Mamba2-8B-shaped SSD layer             (c4)
  Mamba2-8B-shaped decode                (c5)
Stream ids: x=0, B=1, C=2, delta=3, A=4, D=5, h0=6, calibration=9 (+10 for B/C calibration);
decode step k draws from ``[5, k, stream]``.
"""
from __future__ import annotations

import numpy as np

X, BS, CS, DT, AS, DS, H0, CAL, CALBC = 0, 1, 2, 3, 4, 5, 6, 9, 10


def rng(cfg, *stream):
    return np.random.default_rng([int(cfg), *[int(s) for s in stream]])


def _softplus(z):
    # input-generation transform (positive step sizes), not part of the method
    return np.log1p(np.exp(-np.abs(z))) + np.maximum(z, 0.0)


def student_t_outliers(r, shape, df=3.0, frac=0.001, factor=100.0):
    """Heavy-tailed activations: Student-t(df) with i.i.d. Bernoulli(frac) entries scaled by factor."""
    x = r.standard_t(df, size=shape)
    mask = r.random(size=shape) < frac
    x = np.where(mask, x * factor, x)
    return x.astype(np.float32)


# ------------------------------------------------------------------------------------------------
# Mamba1 selective scan layer (c1, c3)

C1 = dict(batch=1, seqlen=256, dim=64, dstate=16, bc_groups=1, gs=4, x_groups=1)
C3 = dict(batch=8, seqlen=2048, dim=1536, dstate=16, bc_groups=1, gs=4, x_groups=8)


def mamba1_inputs(cfg=1, batch=1, seqlen=256, dim=64, dstate=16, bc_groups=1, x_dist="normal",
                  calib_batch=None, with_h0=False, **_):
    """x, delta [B, D, L]; A [D, N]; B, C [B, Gbc, N, L]; D [D]; optional h0 [B, D, N];
    calibration draws x_cal [Bc, D, L], B_cal, C_cal [Bc, Gbc, N, L] (separate streams)."""
    shp = (batch, dim, seqlen)
    bshp = (batch, bc_groups, dstate, seqlen)
    if x_dist == "normal":
        x = rng(cfg, X).standard_normal(shp).astype(np.float32)
    else:
        x = student_t_outliers(rng(cfg, X), shp)
    out = dict(
        x=x,
        B=rng(cfg, BS).standard_normal(bshp).astype(np.float32),
        C=rng(cfg, CS).standard_normal(bshp).astype(np.float32),
        delta=_softplus(rng(cfg, DT).normal(-1.0, 0.5, size=shp)).astype(np.float32),
        A=(-np.exp(rng(cfg, AS).uniform(-1.0, 1.0, size=(dim, dstate)))).astype(np.float32),
        D=rng(cfg, DS).standard_normal(dim).astype(np.float32),
    )
    if with_h0:
        out["h0"] = (0.5 * rng(cfg, H0).standard_normal((batch, dim, dstate))).astype(np.float32)
    if calib_batch:
        cshp = (calib_batch, dim, seqlen)
        rc = rng(cfg, CAL)
        out["x_cal"] = (rc.standard_normal(cshp).astype(np.float32) if x_dist == "normal"
                        else student_t_outliers(rc, cshp))
        rcb = rng(cfg, CALBC)
        cb = (calib_batch, bc_groups, dstate, seqlen)
        out["B_cal"] = rcb.standard_normal(cb).astype(np.float32)
        out["C_cal"] = rcb.standard_normal(cb).astype(np.float32)
    return out


def c1_inputs():
    return mamba1_inputs(cfg=1, **C1)


def c3_inputs(batch=C3["batch"], seqlen=C3["seqlen"], dim=C3["dim"], calib_batch=1):
    return mamba1_inputs(cfg=3, batch=batch, seqlen=seqlen, dim=dim, dstate=16, bc_groups=1,
                         x_dist="student_t", calib_batch=calib_batch)


# ------------------------------------------------------------------------------------------------
# S4D layer (c2)

C2 = dict(batch=16, seqlen=784, channels=128, dstate=64)


def s4d_inputs(cfg=2, batch=16, seqlen=784, channels=128, dstate=64, with_h0=False, **_):
    """pixel sequence p [B, L] ~ U(0,1); lift weights w [H] ~ N(0,1);
    A = -0.5 + i*pi*n (S4D-Lin initialisation) [H, N]; B = 1; C ~ N(0,1) + i N(0,1) [H, N];
    log_dt ~ U(log 1e-3, log 1e-1) [H]; D ~ N(0,1) [H]."""
    H, N = channels, dstate
    n = np.arange(N, dtype=np.float64)
    r = rng(cfg, CS)
    out = dict(
        u=rng(cfg, X).uniform(0.0, 1.0, size=(batch, seqlen)).astype(np.float32),
        w=rng(cfg, BS).standard_normal(H).astype(np.float32),
        A_re=np.full((H, N), -0.5, dtype=np.float32),
        A_im=np.broadcast_to((np.pi * n).astype(np.float32), (H, N)).copy(),
        B_re=np.ones((H, N), dtype=np.float32),
        B_im=np.zeros((H, N), dtype=np.float32),
        C_re=r.standard_normal((H, N)).astype(np.float32),
        C_im=r.standard_normal((H, N)).astype(np.float32),
        log_dt=rng(cfg, DT).uniform(np.log(1e-3), np.log(1e-1), size=H).astype(np.float32),
        D=rng(cfg, DS).standard_normal(H).astype(np.float32),
    )
    if with_h0:
        r0 = rng(cfg, H0)
        out["h0_re"] = (0.1 * r0.standard_normal((batch, H, N))).astype(np.float32)
        out["h0_im"] = (0.1 * r0.standard_normal((batch, H, N))).astype(np.float32)
    return out


# ------------------------------------------------------------------------------------------------
# Mamba2 SSD layer (c4) and decode (c5)

C4 = dict(batch=4, seqlen=4096, nheads=128, headdim=64, dstate=128, ngroups=8, chunk=256, gs=16,
          x_groups_per_block=8)
C5 = dict(batch=256, nheads=128, headdim=64, dstate=128, ngroups=8, gs=16, x_groups_per_block=8,
          steps=64)


def ssd_inputs(cfg=4, batch=4, seqlen=4096, nheads=128, headdim=64, dstate=128, ngroups=8,
               calib_len=None, with_h0=False, **_):
    """x [B, L, nh, P] ~ N(0,1); B, C [B, L, Gbc, N] ~ N(0,1); delta = softplus(N(-2, 0.5))
    [B, L, nh]; A = -exp(U(0, 2)) [nh]; D ~ N(0,1) [nh]; calibration draws of length calib_len."""
    xs = (batch, seqlen, nheads, headdim)
    bs = (batch, seqlen, ngroups, dstate)
    out = dict(
        x=rng(cfg, X).standard_normal(xs, dtype=np.float32),
        B=rng(cfg, BS).standard_normal(bs, dtype=np.float32),
        C=rng(cfg, CS).standard_normal(bs, dtype=np.float32),
        delta=_softplus(rng(cfg, DT).normal(-2.0, 0.5, size=(batch, seqlen, nheads))
                        ).astype(np.float32),
        A=(-np.exp(rng(cfg, AS).uniform(0.0, 2.0, size=nheads))).astype(np.float32),
        D=rng(cfg, DS).standard_normal(nheads).astype(np.float32),
    )
    if with_h0:
        out["h0"] = (0.5 * rng(cfg, H0).standard_normal((batch, nheads, headdim, dstate))
                     ).astype(np.float32)
    if calib_len:
        rc = rng(cfg, CAL)
        out["x_cal"] = rc.standard_normal((1, calib_len, nheads, headdim), dtype=np.float32)
        rcb = rng(cfg, CALBC)
        out["B_cal"] = rcb.standard_normal((1, calib_len, ngroups, dstate), dtype=np.float32)
        out["C_cal"] = rcb.standard_normal((1, calib_len, ngroups, dstate), dtype=np.float32)
    return out


def decode_params(cfg=5, nheads=128, headdim=64, dstate=128, ngroups=8, batch=256, **_):
    """Per-layer decode parameters: A [nh], D [nh], initial state [B, nh, P, N] (0.1*N(0,1)),
    and a calibration draw of one step's x, B, C."""
    r = rng(cfg, AS)
    return dict(
        A=(-np.exp(r.uniform(0.0, 2.0, size=nheads))).astype(np.float32),
        D=rng(cfg, DS).standard_normal(nheads).astype(np.float32),
        state0=(0.1 * rng(cfg, H0).standard_normal((batch, nheads, headdim, dstate),
                                                   dtype=np.float32)),
        x_cal=rng(cfg, CAL).standard_normal((batch, nheads, headdim), dtype=np.float32),
        B_cal=rng(cfg, CALBC).standard_normal((batch, ngroups, dstate), dtype=np.float32),
        C_cal=rng(cfg, CALBC + 1).standard_normal((batch, ngroups, dstate), dtype=np.float32),
    )


def decode_step_inputs(k, cfg=5, batch=256, nheads=128, headdim=64, dstate=128, ngroups=8, **_):
    """Inputs of decode step k: x [B, nh, P], B, C [B, Gbc, N] ~ N(0,1);
    delta = softplus(N(-2, 0.5)) [B, nh]."""
    return dict(
        x=rng(cfg, k, X).standard_normal((batch, nheads, headdim), dtype=np.float32),
        B=rng(cfg, k, BS).standard_normal((batch, ngroups, dstate), dtype=np.float32),
        C=rng(cfg, k, CS).standard_normal((batch, ngroups, dstate), dtype=np.float32),
        delta=_softplus(rng(cfg, k, DT).normal(-2.0, 0.5, size=(batch, nheads))).astype(np.float32),
    )


# ------------------------------------------------------------------------------------------------
# Adversarial quantizer inputs

def quantizer_edge_values(cfg=7, n=4096, scale=np.float32(0.0371)):
    """fp32 values around the rounding ties of scale `scale`: exact half-integer multiples, their
    fp32 neighbours, saturation boundaries, signed zeros, NaN and infinities, and random values."""
    r = rng(cfg, X)
    k = r.integers(-140, 140, size=n).astype(np.float64)
    ties = (k + 0.5) * float(scale)
    t32 = ties.astype(np.float32)
    up = np.nextafter(t32, np.float32(np.inf))
    dn = np.nextafter(t32, np.float32(-np.inf))
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 127.5 * float(scale),
                        -128.5 * float(scale), 126.5 * float(scale), -127.5 * float(scale),
                        1e30, -1e30, 1e-30, -1e-30], dtype=np.float32)
    rand = (r.standard_normal(n) * 60.0 * float(scale)).astype(np.float32)
    return np.concatenate([t32, up, dn, special, rand]).astype(np.float32)


# ------------------------------------------------------------------------------------------------
# W4A8 linear layer (the Mamba2-8B input projection: K = d_model 4096, N = 18560)

def w4a8_inputs(cfg=8, M=256, N=18560, K=4096):
    """Weights w [N, K] ~ N(0, 1/K) with a per-output-channel spread exp(U(-1, 1)); activations x
    [M, K] ~ N(0,1) with 0.1% outliers x10; a calibration draw of the same law [256, K]; bias
    [N] ~ 0.1 N(0,1)."""
    r = rng(cfg, BS)
    w = (r.standard_normal((N, K), dtype=np.float32) / np.float32(np.sqrt(K)) *
         np.exp(rng(cfg, AS).uniform(-1.0, 1.0, (N, 1))).astype(np.float32))
    def act(rr, shape):
        a = rr.standard_normal(shape, dtype=np.float32)
        return np.where(rr.random(shape) < 0.001, a * np.float32(10.0), a).astype(np.float32)
    return dict(w=w.astype(np.float32), x=act(rng(cfg, X), (M, K)), x_cal=act(rng(cfg, CAL), (256, K)),
                bias=(0.1 * rng(cfg, DS).standard_normal(N)).astype(np.float32))
