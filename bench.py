"""Benchmark of the quantized state-space hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only] [--no-cpu-baseline]

One step = one pass of the whole hot path of the workload over one batch of synthetic input that is
already resident in HBM: for the SSD layer (the default, the largest configuration: Mamba2-8B-shaped,
B 4, L 4096, 128 heads x 64, N 128, 8 groups), quantize x, B and C, then run the chunked SSD; for
the Mamba1 layers, quantize x (gathered into cluster order), quantize B and C, run the W8A8 scan;
for S4D, quantize the input then scan; for decode, one fused state update of every sequence.

Per workload, in order:
  1. one step on the GPU;
  2. the oracle on a bounded sample of the same workload, repeated for a few seconds: its rate is
     the cpu_baseline, and its result is the parity reference;
  3. the parity gate: codes bit-exact, outputs of the sample within the stated tolerance (the
     process exits with status 3 on a mismatch, before any timing);
  4. W warmup and K timed steps; `value` from the wall clock over the K steps, and HIP events on the
     launch stream around every 2nd call of the dominant entry point (mean for the roofline,
     median and min reported).

Prints one JSON line. Unless --only is given it also carries the other configurations
(other_configs), each with its own parity result, roofline and cpu_baseline, and a row for the
quantizers alone with the soft-edge / int8 encode ratio.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# fp32 vector peak of MI355X as lane-operations per second: the published 157.3 TFLOP/s counts a
# fused multiply-add as two flops, so 78.6 T FMA lane-ops/s (256 CUs x 4 SIMDs x 32 lanes per clock
# x 2.4 GHz). The instruction-rate probe measures plain (unpacked) v_fma_f32 above the 16-lane
# figure (256 x 4 x 16 x 2.4 GHz = 39.3 T/s), so that figure is no ceiling; v_exp_f32 issues at
# about a quarter of the FMA rate.
VALU_PEAK_TOPS = 157.3 / 2
METRIC = "quantized scan state-updates/s (B·L·D·N) + % of HBM peak, 1 MI355X"


class ParityError(RuntimeError):
    pass


def row_error(y, ref, axis=-1):
    """Per-row normwise error max|y - r| / max(max|r|, 1e-6 max_all|r|) (complex: modulus)."""
    y = np.asarray(y)
    ref = np.asarray(ref)
    dt = np.complex128 if (np.iscomplexobj(y) or np.iscomplexobj(ref)) else np.float64
    y = y.astype(dt)
    ref = ref.astype(dt)
    floor = 1e-6 * max(np.abs(ref).max(initial=0.0), 1e-300)
    return np.abs(y - ref).max(axis=axis) / np.maximum(np.abs(ref).max(axis=axis), floor)


def require(cond, what):
    if not cond:
        raise ParityError(what)


def codes_equal(got, want, name):
    got = np.asarray(got)
    want = np.asarray(want)
    require(got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}")
    n = int(np.count_nonzero(got.view(np.uint8) != want.view(np.uint8)))
    require(n == 0, f"{name}: {n} codes differ")
    return int(got.size)


def rows_close(got, want, tol, name, axis=-1):
    e = float(row_error(got, want, axis=axis).max(initial=0.0))
    require(e <= tol, f"{name}: max row error {e:.3e} above {tol:g}")
    return e


# ------------------------------------------------------------------------------------------------
# workloads

class Workload:
    name = ""
    dominant = ""           # the entry point timed for the roofline
    bound = "hbm"
    tol = 2e-3
    config: dict = {}
    sample_desc = ""

    def setup(self, dev): ...
    def step(self, timer): ...
    def updates(self): ...
    def dominant_bytes(self): ...
    def oracle_ref(self): ...          # the oracle on the sample (timed as the cpu baseline)
    def sample_updates(self): ...      # state updates the sample computes
    def check(self, ref): ...          # parity of the GPU state after the first step


class Mamba1(Workload):
    # per state update: v_mul (delta * A log2 e), v_exp_f32, v_mul (delta x * B), two FMAs (state
    # and readout)
    ops_per_update = 5

    def __init__(self, soft_edge=False, y_int8=False, ratio=4, bc_soft_edge=False, time_blocks=0):
        self.soft = soft_edge
        self.y_int8 = y_int8
        self.ratio = ratio
        self.bc_soft = bc_soft_edge
        self.time_blocks = time_blocks
        self.name = ("mamba1-130m-layer-w8a8" + ("-softedge-x" if soft_edge else "") +
                     ("-shift" if ratio == 2 else "") + ("-softedge-bc" if bc_soft_edge else "") +
                     ("-int8-y" if y_int8 else "") +
                     (f"-{time_blocks}-time-windows" if time_blocks > 1 else ""))
        self.dominant = "qssm_scan_w8a8: k_stage_bc + k_scan_m1"
        self.bound = "alu"

    def setup(self, dev):
        import qssm_synth as synth
        import quantized_state_space_amd as qs
        import quantized_state_space_amd.workloads as wl
        self.inp = synth.c3_inputs()
        form = qs.QSSM_X_SOFTEDGE2 if self.ratio == 2 else qs.QSSM_X_SOFTEDGE
        xc = form if self.soft else qs.QSSM_X_INT8
        bc = form if self.bc_soft else qs.QSSM_X_INT8
        y_out = None
        if self.y_int8:
            # int8 output for the next W8A8 module: 8 clustered output groups calibrated on one
            # fp32-output pass, and a seeded per-channel correction term (~1% of a channel's range)
            import torch
            cal = wl.Mamba1Layer(self.inp, 8, 4, dev, x_code=xc)
            cal.step()
            y = cal.y.cpu().numpy()
            del cal
            torch.cuda.empty_cache()
            yg, ys = wl.calib_y_groups(y, 8)
            ch = qs.qssm_calib_channel_absmax(y)
            yb = (synth.rng(3, 12).standard_normal(ch.size) * 0.01 * ch).astype(np.float32)
            y_out = (yg, ys, yb)
        self.y_out = y_out
        # two copies of every buffer, used in turn, so that one step's 350 MB of traffic cannot be
        # served from the previous step's lines in the 256 MB last-level cache
        self.layers = [wl.Mamba1Layer(self.inp, 8, 4, dev, x_code=xc, y_out=y_out, bc_code=bc,
                                      time_blocks=self.time_blocks) for _ in range(2)]
        self.k = 0
        B, D, L, N, Gbc = self.layers[0].shape
        self.dims = (B, D, L, N, Gbc)
        self.config = {"workload": self.name, "batch": B, "seqlen": L, "d_inner": D, "d_state": N,
                       "x_groups": 8,
                       "x_code": (f"soft-edge 3-scale u8, ratio {self.ratio}" if self.soft
                                  else "int8"),
                       "bc_code": (f"soft-edge 3-scale u8, ratio {self.ratio}" if self.bc_soft
                                   else "int8"),
                       "bc_state_groups": N // 4, "state": "f32",
                       "y": "int8, 8 output groups + per-channel correction" if self.y_int8
                       else "f32"}
        self.sample_desc = "full workload (8 x 1536 channels x 2048 steps): quantize, dequantize, fp64 scan"

    def step(self, timer):
        lay = self.layers[self.k % len(self.layers)]
        self.k += 1
        lay.quantize()
        timer.start()
        lay.scan()
        timer.stop()

    def updates(self):
        B, D, L, N, _ = self.dims
        return B * D * L * N

    sample_updates = updates

    def ops(self):
        return self.ops_per_update * self.updates()

    def dominant_bytes(self):
        B, D, L, N, Gbc = self.dims
        # x codes, delta, B/C codes, A, D in; y and h_last out (each once); an int8 y adds the
        # output groups, scales and correction terms
        yb = 1 if self.y_int8 else 4
        extra = (D + 4 * 8 + 4 * D) if self.y_int8 else 0
        return (B * D * L * (1 + 4 + yb) + 2 * B * Gbc * N * L + 4 * D * N + 4 * D + 4 * B * D * N
                + extra)

    def oracle_ref(self):
        import oracle.pipelines as op
        if not hasattr(self, "_cal"):
            self._cal = op.mamba1_calib(self.inp, 8, 4, soft_edge=self.soft,
                                        bc_soft_edge=self.bc_soft)
        return op.mamba1(self.inp, G=8, gs=4, soft_edge=self.soft, calib=self._cal,
                         se_ratio=self.ratio, bc_soft_edge=self.ratio if self.bc_soft else 0)

    def check(self, ref):
        lay = self.layers[0]  # ran the first step
        n = codes_equal(lay.xq.cpu().numpy(), ref["xq"], "x codes")
        n += codes_equal(lay.Bq.cpu().numpy().view(np.uint8), ref["Bq"].view(np.uint8), "B codes")
        n += codes_equal(lay.Cq.cpu().numpy().view(np.uint8), ref["Cq"].view(np.uint8), "C codes")
        out = {"codes_bit_exact": n}
        out["h_last_row_error"] = rows_close(lay.h_last.cpu().numpy(), ref["h_last"], self.tol,
                                             "h_last")
        if not self.y_int8:
            out["y_row_error"] = rows_close(lay.y.float().cpu().numpy(), ref["y"], self.tol, "y")
        else:
            # decode the int8 codes with the static output scales and correction term: every
            # unsaturated code is within half a step (plus the fp32-state tolerance of the row) of
            # the oracle's y + bias
            yg, ys, yb = self.y_out
            codes = lay.y.cpu().numpy().astype(np.float64)
            s = np.asarray(ys, np.float64)[np.asarray(yg, np.int64)][None, :, None]
            v = np.asarray(ref["y"], np.float64) + np.asarray(yb, np.float64)[None, :, None]
            inside = (codes > -128) & (codes < 127)
            rowmax = np.abs(ref["y"]).max(axis=-1, keepdims=True)
            dev = np.abs(codes * s - v) - (0.5 * s + self.tol * rowmax)
            bad = int(np.count_nonzero((dev > 1e-9 * s) & inside))
            require(bad == 0, f"int8 y: {bad} codes off by more than half a step")
            out["y_int8_codes_within_half_step"] = int(np.count_nonzero(inside))
        return out


class Tiny(Mamba1):
    """time_blocks: 0 = the library's choice (time windows at this size), 1 = one chain per state
    in time order."""
    def __init__(self, time_blocks=0):
        self.soft = False
        self.y_int8 = False
        self.time_blocks = time_blocks
        self.name = "tiny-mamba1-w8a8" + ("-chain-form" if time_blocks == 1 else "")
        self.dominant = ("qssm_scan_w8a8: k_stage_bc + k_scan_m1" if time_blocks == 1 else
                         "qssm_scan_w8a8: k_stage_bc + k_scan_m1 (window states) + k_scan_carry "
                         "+ k_scan_m1 (windows)")
        self.bound = "alu"

    def setup(self, dev):
        import qssm_synth as synth
        import quantized_state_space_amd.workloads as wl
        self.inp = synth.c1_inputs()
        self.layers = [wl.Mamba1Layer(self.inp, 1, 4, dev, dynamic_scales=True,
                                      time_blocks=self.time_blocks)]
        self.k = 0
        self.dims = self.layers[0].shape
        B, D, L, N, _ = self.dims
        self.config = {"workload": self.name, "batch": B, "seqlen": L, "d_inner": D, "d_state": N,
                       "x_groups": 1, "bc_state_groups": 4, "state": "f32", "y": "f32",
                       "scan_form": "chain" if self.time_blocks == 1 else
                       "library choice (time windows)"}
        self.sample_desc = "full workload, on-device scales"

    def oracle_ref(self):
        import oracle.pipelines as op
        return op.mamba1(self.inp, G=1, gs=4, dynamic=True)


class S4d(Workload):
    # per complex state update, in the cheapest form the kernel uses (the chain on g = h / Bbar'):
    # Abar g + q (4 FMA-class) and Re(C' g) (2 FMA-class)
    ops_per_update = 6

    def __init__(self, i16=False):
        self.i16 = i16
        self.name = "s4d-smnist-shaped" + ("-int16-state" if i16 else "")
        self.dominant = "qssm_s4d_scan: k_s4d"
        self.bound = "alu"
        self.tol = 1e-2 if i16 else 2e-3

    def setup(self, dev):
        import qssm_synth as synth
        import quantized_state_space_amd as qs
        import quantized_state_space_amd.workloads as wl
        self.inp = synth.s4d_inputs()
        # int16 state: the per-channel scale from the library's host calibration (the recurrence's
        # geometric bound on the quantized parameters)
        self.lay = wl.S4dLayer(self.inp, dev, state_dtype=qs.QSSM_I16 if self.i16 else qs.QSSM_F32)
        B, L, H, N = self.lay.shape
        self.dims = (B, L, H, N)
        self.config = {"workload": self.name, "batch": B, "seqlen": L, "channels": H,
                       "d_state_complex": N, "state": "int16" if self.i16 else "f32", "y": "f32"}
        self.sample_desc = "full workload, fp64 complex scan" + (
            " with the same int16 state grid" if self.i16 else "")

    def step(self, timer):
        import quantized_state_space_amd as qs
        qs.qssm_quant_group_x(self.lay.u_f, _zero(self.lay.u_f.device), 1, self.lay.u_scale,
                              self.lay.uq)
        timer.start()
        qs.qssm_s4d_scan(self.lay.args)
        timer.stop()

    def updates(self):
        B, L, H, N = self.dims
        return B * L * H * N

    sample_updates = updates

    def ops(self):
        return self.ops_per_update * self.updates()

    def dominant_bytes(self):
        B, L, H, N = self.dims
        sb = 4 if self.i16 else 8
        return B * L + H + 6 * H * N + 4 * 8 * H + 4 * B * H * L + sb * B * H * N

    def oracle_ref(self):
        import oracle.pipelines as op
        return op.s4d(self.inp, state_scale=self.lay.state_scale_host if self.i16 else None)

    def check(self, ref):
        out = {"codes_bit_exact": codes_equal(self.lay.uq.cpu().numpy()[:, 0, :], ref["uq"],
                                              "input codes")}
        out["y_row_error"] = rows_close(self.lay.y.cpu().numpy(), ref["y"], self.tol, "y")
        if not self.i16:
            hl = self.lay.h_last.cpu().numpy()
            out["h_last_row_error"] = rows_close(hl[..., 0] + 1j * hl[..., 1], ref["h_last"],
                                                 self.tol, "h_last")
        return out


# Near-boundary margin of the int8 intra-chunk codes: the kernel forms W from G carried in fp16
# (2^-11) and decides its row scale from that W (2^-11 again), decay factors ~1e-5.
INTRA8_EPS_REL, INTRA8_EPS_ABS = 1.2e-3, 1e-4


class Ssd(Workload):
    def __init__(self, f16=False, y_int8=False, intra8=False):
        self.f16 = f16
        self.y_int8 = y_int8
        self.intra8 = intra8
        self.name = ("mamba2-8b-ssd-layer-w8a8" + ("-fp16-y" if f16 else "") +
                     ("-int8-y" if y_int8 else "") + ("-int8-intra" if intra8 else ""))
        self.dominant = "qssm_ssd_chunk_int8: k_ssd_state + k_ssd_output"
        self.heads = np.array([0, 64])

    def setup(self, dev):
        import qssm_synth as synth
        import quantized_state_space_amd as qs
        import quantized_state_space_amd.workloads as wl
        self.inp = synth.ssd_inputs(cfg=4, calib_len=256)
        y_out = None
        if self.y_int8:
            # int8 output for the next W8A8 module: 8 clustered output groups per head block,
            # calibrated on one fp32-output pass, and a seeded per-channel correction term (~1% of
            # a channel's range)
            import torch
            cal = wl.SsdLayer(self.inp, dev)
            cal.step()
            B, L, nh, P, N, Gbc = cal.shape
            y = cal.y.cpu().numpy().reshape(B * L, nh * P)
            del cal
            torch.cuda.empty_cache()
            yg, ys = wl.calib_ssd_x_groups(y, nh, P, Gbc, 8)
            ch = qs.qssm_calib_channel_absmax(y.reshape(B * L, nh * P, 1))
            yb = (synth.rng(4, 12).standard_normal(ch.size) * 0.01 * ch).astype(np.float32)
            y_out = (yg, ys, yb)
        self.y_out = y_out
        self.lay = wl.SsdLayer(self.inp, dev, y_dtype=qs.QSSM_F16 if self.f16 else qs.QSSM_F32,
                               y_out=y_out,
                               intra_mma=qs.QSSM_MMA_I8 if self.intra8 else qs.QSSM_MMA_F16)
        B, L, nh, P, N, Gbc = self.lay.shape
        self.dims = self.lay.shape
        self.config = {"workload": self.name, "batch": B, "seqlen": L, "heads": nh, "headdim": P,
                       "d_state": N, "ngroups": Gbc, "chunk": 256, "x_groups": int(self.lay.G),
                       "bc_state_groups": N // 16, "state": "f32",
                       "y": "int8, 8 output groups per head block + per-channel correction"
                       if self.y_int8 else ("f16" if self.f16 else "f32"),
                       "intra_chunk": "int8 MFMA, row-requantized weights" if self.intra8
                       else "fp16 MFMA"}
        self.sample_desc = (f"{len(self.heads)} of {nh} heads (all batches, full length): the fp64 "
                            "chunked form, including quantizing the layer's whole x, B and C")

    def step(self, timer):
        self.lay.quantize()
        timer.start()
        self.lay.scan()
        timer.stop()

    def updates(self):
        B, L, nh, P, N, _ = self.dims
        return B * L * nh * P * N

    def sample_updates(self):
        B, L, nh, P, N, _ = self.dims
        return B * L * len(self.heads) * P * N

    def mfma_ops(self):
        """Algorithmic matrix ops of the dominant call by operand type (multiply-add = 2, causal
        halves counted once): C B^T in int8 per (b, chunk, group); the intra-chunk product, the
        chunk state and the inter-chunk product per (b, chunk, head). Peak: dense MFMA T ops/s."""
        B, L, nh, P, N, Gbc = self.dims
        nc = -(-L // 256)
        tri = 256 * 257 // 2
        cb = 2 * B * nc * Gbc * tri * N
        intra = 2 * B * nc * nh * tri * P
        state = 2 * B * nc * nh * 256 * P * N
        inter = 2 * B * nc * nh * 256 * N * P
        i8 = cb + (intra if self.intra8 else 0)
        f16 = state + inter + (0 if self.intra8 else intra)
        return {"int8": (INT8_MFMA_PEAK_TOPS, i8), "fp16": (FP16_MFMA_PEAK_TFLOPS, f16)}

    def dominant_bytes(self):
        B, L, nh, P, N, Gbc = self.dims
        yb = 1 if self.y_int8 else (2 if self.f16 else 4)
        # x codes, delta, B/C codes, A, D in; y out; h_last out (each once)
        return B * L * nh * P * (1 + yb) + 4 * B * L * nh + 2 * B * L * Gbc * N + 8 * nh + \
            4 * B * nh * P * N

    def oracle_ref(self):
        import oracle.pipelines as op
        return op.ssd(self.inp, heads=self.heads, int8_intra=self.intra8)

    def check(self, ref):
        lay = self.lay
        n = codes_equal(lay.xq.cpu().numpy(), ref["xq"], "x codes")
        n += codes_equal(lay.Bq.cpu().numpy().view(np.uint8), ref["Bq"].view(np.uint8), "B codes")
        n += codes_equal(lay.Cq.cpu().numpy().view(np.uint8), ref["Cq"].view(np.uint8), "C codes")
        import torch
        hsel = torch.as_tensor(self.heads, device=lay.y.device)
        rows = lambda a: np.asarray(a, np.float64).transpose(0, 2, 3, 1).reshape(-1, a.shape[1])
        out = {"codes_bit_exact": n}
        if self.intra8:
            # each output within the row tolerance plus one requantization step times |xh_j| for
            # every weight code of its row that lies within the kernel's error of a boundary
            import oracle.pipelines as op
            y = rows(lay.y[:, :, hsel].float().cpu().numpy())
            yr = rows(ref["y"])
            slack, near, total = op.ssd_intra_near_boundary(self.inp, ref, INTRA8_EPS_REL,
                                                            INTRA8_EPS_ABS)
            allow = self.tol * np.abs(yr).max(axis=1, keepdims=True) + rows(slack)
            used = float(np.max(np.abs(y - yr) / allow))
            require(used <= 1.0, f"int8 intra-chunk y beyond its allowance ({used:.3f})")
            out["y_within_allowance"] = round(used, 4)
            out["near_boundary_codes"] = f"{near} of {total}"
        elif not self.y_int8:
            y = lay.y[:, :, hsel].float().cpu().numpy().astype(np.float64)
            out["y_row_error"] = rows_close(rows(y), rows(ref["y"]), self.tol, "y")
        else:
            # decode the int8 codes with the static output scales and correction term: every
            # unsaturated code is within half a step (plus the fp32-state tolerance of the row) of
            # the oracle's y + bias
            yg, ys, yb = self.y_out
            P = self.dims[3]
            ch = (self.heads[:, None] * P + np.arange(P)[None, :]).reshape(-1)
            codes = rows(lay.y[:, :, hsel].cpu().numpy().astype(np.float64))
            yr = rows(ref["y"])
            nrow = yr.shape[0] // len(ch)                      # rows are (b, head, p)
            s = np.tile(np.asarray(ys, np.float64)[np.asarray(yg, np.int64)][ch], nrow)[:, None]
            v = yr + np.tile(np.asarray(yb, np.float64)[ch], nrow)[:, None]
            inside = (codes > -128) & (codes < 127)
            rowmax = np.abs(yr).max(axis=-1, keepdims=True)
            dev = np.abs(codes * s - v) - (0.5 * s + self.tol * rowmax)
            bad = int(np.count_nonzero((dev > 1e-9 * s) & inside))
            require(bad == 0, f"int8 y: {bad} codes off by more than half a step")
            out["y_int8_codes_within_half_step"] = int(np.count_nonzero(inside))
        hl = lay.h_last[:, hsel].cpu().numpy()
        out["h_last_row_error"] = rows_close(hl.reshape(-1, hl.shape[-1]),
                                             ref["h_last"].reshape(-1, hl.shape[-1]), self.tol,
                                             "h_last")
        return out


class Decode(Workload):
    def __init__(self, f16=False):
        self.f16 = f16
        self.name = "mamba2-8b-decode" + ("-fp16-state" if f16 else "")
        self.dominant = "qssm_state_update: k_state_update"
        self.tol = 1e-2 if f16 else 2e-3
        self.sample = np.array([0, 77, 130, 255])
        self.base_sample = np.arange(16)

    def setup(self, dev):
        import torch
        import qssm_synth as synth
        import quantized_state_space_amd as qs
        import quantized_state_space_amd.workloads as wl
        self.params = synth.decode_params()
        if self.f16:  # the fp16 state starts from the fp16-rounded initial state on both sides
            self.params["state0"] = self.params["state0"].astype(np.float16).astype(np.float32)
        self.lay = wl.DecodeLayer(self.params, dev, state_dtype=qs.QSSM_F16 if self.f16 else qs.QSSM_F32)
        B, nh, P, N, Gbc = self.lay.shape
        self.dims = self.lay.shape
        self.nsteps = 64
        self.inputs = [synth.decode_step_inputs(k) for k in range(self.nsteps)]
        # all 64 tokens resident in HBM; one argument block per token (the first also publishes the
        # codes, for the parity gate)
        self.codes = (torch.empty((B, nh, P), dtype=torch.int8, device=dev),
                      torch.empty((B, Gbc, N), dtype=torch.int8, device=dev),
                      torch.empty((B, Gbc, N), dtype=torch.int8, device=dev))
        self.dev_inputs = []
        self.args = []
        for k, inp in enumerate(self.inputs):
            d = {n: torch.from_numpy(inp[n]).to(dev) for n in ("x", "B", "C", "delta")}
            self.dev_inputs.append(d)
            self.args.append(qs.update_args(d["x"], self.lay.group_t, self.lay.xs, d["B"], d["C"],
                                            self.lay.bs, self.lay.cs, 16, d["delta"], self.lay.A,
                                            self.lay.state, self.lay.y, Dskip=self.lay.D))
        d = self.dev_inputs[0]
        self.gate_args = qs.update_args(d["x"], self.lay.group_t, self.lay.xs, d["B"], d["C"],
                                        self.lay.bs, self.lay.cs, 16, d["delta"], self.lay.A,
                                        self.lay.state, self.lay.y, Dskip=self.lay.D,
                                        xq_out=self.codes[0], Bq_out=self.codes[1],
                                        Cq_out=self.codes[2])
        self.k = 0
        self.config = {"workload": self.name, "batch": B, "heads": nh, "headdim": P, "d_state": N,
                       "ngroups": Gbc, "tokens": self.nsteps, "state": "f16" if self.f16 else "f32"}
        self.sample_desc = (f"{len(self.base_sample)} of {B} sequences x 8 tokens, fp64 state "
                            "(parity: the first token of 4 sequences, codes of all 256)")

    def step(self, timer):
        import quantized_state_space_amd as qs
        timer.start()
        qs.qssm_state_update(self.gate_args if self.k == 0 else self.args[self.k % self.nsteps])
        timer.stop()
        self.k += 1

    def updates(self):
        B, nh, P, N, _ = self.dims
        return B * nh * P * N

    def sample_updates(self):
        B, nh, P, N, _ = self.dims
        return 8 * len(self.base_sample) * nh * P * N

    def dominant_bytes(self):
        B, nh, P, N, Gbc = self.dims
        sb = 2 if self.f16 else 4
        return 2 * sb * B * nh * P * N + 4 * (2 * B * nh * P + 2 * B * Gbc * N + B * nh)

    def oracle_ref(self):
        import oracle.pipelines as op
        op.decode(self.params, self.inputs[:8], batches=self.base_sample)  # the timed sample
        return op.decode(self.params, self.inputs[:1], batches=self.sample)

    def check(self, ref):
        import oracle
        B, nh, P, N, Gbc = self.dims
        inp = self.inputs[0]
        # codes of every sequence for the first token, by the oracle's quantizer and calibration
        xq = oracle.quant_group_x(inp["x"].reshape(B, nh * P, 1), ref["group_of"],
                                  ref["xs"]).reshape(B, nh, P)
        Bq = oracle.quant_state_group(inp["B"][..., None], 16, ref["bs"])[..., 0]
        Cq = oracle.quant_state_group(inp["C"][..., None], 16, ref["cs"])[..., 0]
        n = codes_equal(self.codes[0].cpu().numpy(), xq, "x codes")
        n += codes_equal(self.codes[1].cpu().numpy(), Bq, "B codes")
        n += codes_equal(self.codes[2].cpu().numpy(), Cq, "C codes")
        import torch
        sel = torch.as_tensor(self.sample, device=self.lay.y.device)
        y = self.lay.y[sel].cpu().numpy()
        st = self.lay.state[sel].float().cpu().numpy()
        return {"codes_bit_exact": n,
                "y_row_error": rows_close(y, ref["y"][0], self.tol, "y"),
                "state_row_error": rows_close(st, ref["state"], self.tol, "state")}


class W4A8(Workload):
    """The W4A8 linear layer on the Mamba2-8B input projection shape (K = 4096 -> N = 18560) at M
    tokens: quantize the fp32 activations to int8 (static per-tensor scale), then the GEMM. Not a
    scan: its rate is int8 ops/s, against the int8 MFMA peak."""
    bound = "mfma"
    tol = 1e-5

    def __init__(self, M):
        self.M = M
        self.name = f"w4a8-mamba2-8b-in-proj-m{M}"
        self.dominant = "qssm_gemm_w4a8: k_gemm_w4a8"
        self.rows = np.array([0, M // 2, M - 1])

    def setup(self, dev):
        import qssm_synth as synth
        import quantized_state_space_amd.workloads as wl
        self.inp = synth.w4a8_inputs(cfg=8, M=self.M)
        self.lay = wl.W4A8Linear(self.inp["w"], self.inp["x"], self.inp["x_cal"], dev,
                                 bias=self.inp["bias"])
        M, N, K = self.lay.shape
        self.dims = (M, N, K)
        self.config = {"workload": self.name, "tokens": M, "in_features": K, "out_features": N,
                       "weights": "int4, one scale per output channel", "activations": "int8",
                       "y": "f32"}
        self.sample_desc = f"{len(self.rows)} of {M} rows x all {N} outputs, exact integer dots in fp64"

    def step(self, timer):
        self.lay.quantize()
        timer.start()
        self.lay.gemm()
        timer.stop()

    def updates(self):
        M, N, K = self.dims
        return 2 * M * N * K   # int8 ops (a multiply-add counts two)

    def sample_updates(self):
        M, N, K = self.dims
        return 2 * len(self.rows) * N * K

    def ops(self):
        return self.updates()

    def dominant_bytes(self):
        M, N, K = self.dims
        return M * K + N * K // 2 + 4 * N * (K // K) + 4 * N + 4 * M * N

    def oracle_ref(self):
        import oracle
        inp = self.inp
        x = inp["x"][self.rows]
        sa = oracle.scale_from_absmax(oracle.finite_absmax(inp["x_cal"].reshape(1, -1), axis=1))[0]
        qa = oracle.quant_group_x(x.reshape(1, 1, -1), np.zeros(1, np.uint8), [sa]).reshape(x.shape)
        K = inp["w"].shape[1]
        sw = oracle.w4_scales(inp["w"], K)
        qw = oracle.quant_w4(inp["w"], K, sw)
        return dict(qa=qa, sw=sw, y=oracle.gemm_w4a8(qa, sa, qw, sw, K,
                                                      inp["bias"].astype(np.float64)))

    def check(self, ref):
        import torch
        sel = torch.as_tensor(self.rows, device=self.lay.y.device)
        n = codes_equal(self.lay.xq[sel].cpu().numpy(), ref["qa"], "activation codes")
        require(np.array_equal(self.lay.w_scales_host, ref["sw"]), "weight scales differ")
        return {"codes_bit_exact": n,
                "y_row_error": rows_close(self.lay.y[sel].cpu().numpy(), ref["y"], self.tol, "y")}


_zc = {}


def _zero(device):
    import torch
    k = str(device)
    if k not in _zc:
        _zc[k] = torch.zeros(1, dtype=torch.uint8, device=device)
    return _zc[k]


WORKLOADS = {"c4": lambda: Ssd(False), "c4f16": lambda: Ssd(True),
             "c4i8y": lambda: Ssd(False, True), "c4i8i": lambda: Ssd(False, False, True),
             "c3": lambda: Mamba1(False),
             "c3se": lambda: Mamba1(True), "c3i8y": lambda: Mamba1(False, True), "c1": Tiny,
             "c3se2bc": lambda: Mamba1(True, ratio=2, bc_soft_edge=True),
             "c1chain": lambda: Tiny(1), "c3w4": lambda: Mamba1(False, time_blocks=4),
             "c2": lambda: S4d(False), "c2i16": lambda: S4d(True), "c5": lambda: Decode(False),
             "c5f16": lambda: Decode(True), "w4a8d": lambda: W4A8(256), "w4a8p": lambda: W4A8(16384)}
OTHERS = ("c1", "c1chain", "c2", "c2i16", "c3", "c3w4", "c3se", "c3se2bc", "c3i8y", "c4f16",
          "c4i8y", "c4i8i", "c5", "c5f16", "w4a8d", "w4a8p")
INT8_MFMA_PEAK_TOPS = 5000.0  # dense int8 MFMA, MI355X
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 MFMA, MI355X


# ------------------------------------------------------------------------------------------------

# HBM traffic of one call of the dominant entry point, from two rocprofv3 counter runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, summed over the call's kernels), each divided by
# the ratio the same counter reads for a plain 1 GiB device copy (bench.py --copy-probe). Keyed by
# workload: (fetch bytes, write bytes, digest of the kernel sources when the counters were taken).
TRAFFIC = {
    "c4": (480808192, 696804650, "19659ed6fdd72e73"),
    "c4f16": (479886421, 427856938, "19659ed6fdd72e73"),
    "c4i8y": (481114794, 294124373, "19659ed6fdd72e73"),
    "c4i8i": (480786346, 696856277, "19659ed6fdd72e73"),
    "c3": (153177301, 134756394, "3cdf3e90c9d61e8b"),
    "c3se": (156280789, 134674357, "3cdf3e90c9d61e8b"),
    "c3i8y": (135517269, 27820032, "3cdf3e90c9d61e8b"),
    "c2": (373760, 7472128, "8dbafe7953cbf0db"),
    "c2i16": (391168, 6947200, "8dbafe7953cbf0db"),
    "c5": (1100235776, 1082524586, "3f9c130349ee8131"),
    "c5f16": (563252224, 545275178, "3f9c130349ee8131"),
    "w4a8p": (1861718101, 1216348160, "6fc507f8368b7514"),
    "c1": (1788928, 221184, "3cdf3e90c9d61e8b"),
    "w4a8d": (47269290, 19005440, "6fc507f8368b7514"),
}
TRAFFIC_SOURCES = {
    "c1": ["scan_m1.hip"], "c3": ["scan_m1.hip"], "c3se": ["scan_m1.hip"],
    "c3se2bc": ["scan_m1.hip"], "c1chain": ["scan_m1.hip"], "c3w4": ["scan_m1.hip"],
    "c3i8y": ["scan_m1.hip"], "c2": ["s4d.hip"], "c2i16": ["s4d.hip"],
    "c4": ["ssd.hip"], "c4f16": ["ssd.hip"], "c4i8y": ["ssd.hip"], "c4i8i": ["ssd.hip"],
    "c5": ["state_update.hip"],
    "c5f16": ["state_update.hip"], "w4a8p": ["gemm_w4a8.hip"], "w4a8d": ["gemm_w4a8.hip"],
}


def sources_digest(workload):
    """Digest of the kernel sources a workload runs, comments and layout removed (a comment edit
    keeps the counters valid; any code change voids them)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[workload] + ["common.hpp"]:
        with open(os.path.join(ROOT, "quantized_state_space_amd", "csrc", f), "r") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """Counter-measured HBM bytes per call, or None when none were taken for these sources."""
    t = TRAFFIC.get(workload)
    if t is None or t[2] != sources_digest(workload):
        return None
    return int(t[0] + t[1])


def copy_probe(torch, dev, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of nbytes, the reference kernel for scaling the counters."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": nbytes, "reps": reps}), flush=True)


class EventTimer:
    """HIP events around the dominant call, recorded on the stream the library launches on, for
    every `every`-th timed call (a pair of event records adds a few us of stream time to the step it
    brackets)."""

    def __init__(self, torch, every=2):
        self.torch = torch
        self.pairs = []
        self.active = False
        self.every = every
        self.calls = 0

    def start(self):
        if self.active and self.calls % self.every == 0:
            e = self.torch.cuda.Event(enable_timing=True)
            e.record(self.torch.cuda.current_stream())
            self.pairs.append([e, None])

    def stop(self):
        if self.active:
            if self.calls % self.every == 0:
                e = self.torch.cuda.Event(enable_timing=True)
                e.record(self.torch.cuda.current_stream())
                self.pairs[-1][1] = e
            self.calls += 1

    def samples_ms(self):
        return np.array([a.elapsed_time(b) for a, b in self.pairs])


class _NoTimer:
    def start(self):
        pass

    def stop(self):
        pass


def cpu_and_parity(wl, budget_s, with_baseline=True):
    """Runs the oracle on the workload's sample (repeated for budget_s for the rate) and gates on
    parity. Returns (cpu_baseline dict or None, parity dict)."""
    import oracle
    t0 = time.perf_counter()
    ref = wl.oracle_ref()
    reps = 1
    while with_baseline and time.perf_counter() - t0 < budget_s:
        wl.oracle_ref()
        reps += 1
    dt = time.perf_counter() - t0
    parity = wl.check(ref)
    parity["tolerance"] = wl.tol
    base = None
    if with_baseline:
        unit = "int8 ops/s" if wl.bound == "mfma" else "state-updates/s"
        base = {"value": reps * wl.sample_updates() / dt, "unit": unit,
                "cores": oracle.max_threads(), "kind": "oracle",
                "sample": f"{wl.sample_desc}; {reps} rep(s) in {dt:.1f} s"}
    return base, parity


def run_workload(torch, dev, name, steps, warmup, budget_s, with_baseline=True):
    """Sets up workload `name`, gates it on parity, runs warmup + timed steps; returns
    (workload, results)."""
    wl = WORKLOADS[name]()
    wl.setup(dev)
    wl.step(_NoTimer())
    torch.cuda.synchronize()
    base, parity = cpu_and_parity(wl, budget_s, with_baseline)
    timer = EventTimer(torch)
    for _ in range(warmup):
        wl.step(timer)
    torch.cuda.synchronize()
    timer.active = True
    t0 = time.perf_counter()
    for _ in range(steps):
        wl.step(timer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    samples = timer.samples_ms()
    kern_ms = float(samples.mean())
    nbytes = wl.dominant_bytes()
    if wl.bound == "alu":
        achieved = wl.ops() / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(achieved, 3), "peak": round(VALU_PEAK_TOPS, 2),
                "unit": "T VALU lane-ops/s", "frac": round(achieved / VALU_PEAK_TOPS, 4)}
    elif wl.bound == "mfma":
        achieved = wl.ops() / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_MFMA_PEAK_TOPS,
                "unit": "T int8 ops/s", "frac": round(achieved / INT8_MFMA_PEAK_TOPS, 4)}
    else:
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(name)
    roof["kernel"] = wl.dominant
    roof["kernel_us"] = round(kern_ms * 1e3, 2)
    roof["kernel_us_median"] = round(float(np.median(samples)) * 1e3, 2)
    roof["kernel_us_min"] = round(float(samples.min()) * 1e3, 2)
    roof["kernel_samples"] = int(samples.size)
    roof["algorithmic_bytes"] = int(nbytes)
    if wl.bound == "alu":
        roof["ops_per_update"] = wl.ops_per_update
    res = {"value": wl.updates() * steps / elapsed, "ms_per_step": elapsed * 1e3 / steps,
           "roofline": roof, "parity": parity,
           "hbm_frac_dominant": round(nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if hasattr(wl, "mfma_ops"):
        res["mfma"] = {k: {"ops": int(v[1]), "T_ops_s": round(v[1] / (kern_ms * 1e-3) / 1e12, 1),
                           "frac_of_dense_peak": round(v[1] / (kern_ms * 1e-3) / 1e12 / v[0], 4)}
                       for k, v in wl.mfma_ops().items()}
    if base is not None:
        res["cpu_baseline"] = base
    return wl, res


def probe_row(torch, dev, reps=5):
    """Instruction-rate loops (qssm_probe_rate): v_exp_f32 alone, v_fma_f32 alone, both
    interleaved (whether the exp co-issues with FMA), and the dense int8 / fp16 MFMA rates,
    event-timed, median of reps, against the peaks used for the rooflines."""
    import quantized_state_space_amd as qs
    blocks, iters, miters = 2048, 4096, 128
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    lanes = blocks * 256
    kinds = {"exp": (qs.QSSM_PROBE_EXP, iters, lanes * iters * 8, "T v_exp_f32/s",
                     VALU_PEAK_TOPS),
             "fma": (qs.QSSM_PROBE_FMA, iters, lanes * iters * 8, "T v_fma_f32/s", VALU_PEAK_TOPS),
             "exp_plus_fma": (qs.QSSM_PROBE_EXP_FMA, iters, lanes * iters * 16,
                              "T VALU instructions/s (half exp, half fma)", VALU_PEAK_TOPS),
             "mfma_i8": (qs.QSSM_PROBE_MFMA_I8, miters, blocks * 4 * miters * 2 * 32768 * 2,
                         "T int8 ops/s", INT8_MFMA_PEAK_TOPS),
             "mfma_f16": (qs.QSSM_PROBE_MFMA_F16, miters, blocks * 4 * miters * 2 * 16384 * 2,
                          "T fp16 flops/s", FP16_MFMA_PEAK_TFLOPS)}
    out = {}
    for name, (kind, iters, ops, unit, peak) in kinds.items():
        qs.qssm_probe_rate(kind, iters, blocks, sink)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            qs.qssm_probe_rate(kind, iters, blocks, sink)
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        t = float(np.median(ts))
        rate = ops / t / 1e12
        out[name] = {"rate": round(rate, 2), "unit": unit, "of_peak": round(rate / peak, 3),
                     "us": round(t * 1e6, 1)}
    out["exp_co_issues_with_fma"] = bool(out["exp_plus_fma"]["us"] <
                                         0.9 * (out["exp"]["us"] + out["fma"]["us"]))
    out["note"] = (f"{blocks} workgroups x 256 threads; VALU peak {VALU_PEAK_TOPS:.1f} T "
                   "lane-ops/s (the published fp32 vector 157.3 TFLOP/s, an FMA as one op); "
                   "MFMA peaks dense")
    return out


def quantizer_row(torch, dev, reps=20):
    """The x quantizers alone on the Mamba1-130M x (8 x 1536 x 2048, cluster gather, 8 groups):
    int8 and soft-edge encode on the same bytes, event-timed, codes checked against the oracle."""
    import oracle
    import qssm_synth as synth
    import quantized_state_space_amd as qs
    import quantized_state_space_amd.workloads as wl
    inp = synth.c3_inputs()
    lay = wl.Mamba1Layer(inp, 8, 4, dev)
    s, Lt, Ht, st0 = wl.calib_softedge(inp["x_cal"], lay.perm, lay.group_of, 8, with_state=True)
    st, Lt_t, Ht_t = (torch.from_numpy(a).to(dev) for a in (s, Lt, Ht))
    code = torch.empty(lay.xq.shape, dtype=torch.uint8, device=dev)
    code2 = torch.empty(lay.xq.shape, dtype=torch.uint8, device=dev)
    # threshold tracking into its own buffers, from the calibration state every call
    ema0 = torch.from_numpy(st0).to(dev)
    ema = ema0.clone()
    ts_, tL, tH = (torch.empty(8, dtype=torch.float32, device=dev) for _ in range(3))
    tws = torch.empty(qs.qssm_softedge_track_workspace_size(8), dtype=torch.uint8, device=dev)

    def track():
        ema.copy_(ema0)
        qs.qssm_softedge_track(lay.x, lay.group_t, 8, ema, ts_, tL, tH, tws, ema_valid=True,
                               perm=lay.perm_t)

    calls = {"int8": lambda: qs.qssm_quant_group_x(lay.x, lay.group_t, 8, lay.xs, lay.xq,
                                                   perm=lay.perm_t),
             "softedge": lambda: qs.qssm_softedge_encode(lay.x, lay.group_t, 8, st, Lt_t, Ht_t,
                                                         code, perm=lay.perm_t),
             "softedge_shift": lambda: qs.qssm_softedge_encode(
                 lay.x, lay.group_t, 8, st, Lt_t, Ht_t, code2, perm=lay.perm_t,
                 form=qs.QSSM_X_SOFTEDGE2),
             "track": track}
    for f in calls.values():
        f()
    torch.cuda.synchronize()
    # parity: the codes of both encoders against the oracle's (with its own calibration), bit for bit
    import oracle.pipelines as op
    perm, group_of, xs = op.calib_x(inp["x_cal"], 8)
    se, se_state = op.calib_softedge(inp["x_cal"], perm, group_of, 8, with_state=True)
    want8 = oracle.quant_group_x(inp["x"], group_of, xs, perm=perm)
    codes_equal(lay.xq.cpu().numpy(), want8, "int8 x codes")
    wantse = oracle.softedge_encode(inp["x"], group_of, se[0], se[1], se[2], perm=perm)
    codes_equal(code.cpu().numpy(), wantse, "soft-edge x codes")
    wantse2 = oracle.softedge_encode(inp["x"], group_of, se[0], se[1], se[2], perm=perm, ratio=2)
    codes_equal(code2.cpu().numpy(), wantse2, "shift-form soft-edge x codes")
    ws_, wL, wH, wst = oracle.softedge_track(inp["x"], group_of, 8, perm=perm, prev=se_state)
    require(np.array_equal(ts_.cpu().numpy(), ws_) and np.array_equal(tL.cpu().numpy(), wL)
            and np.array_equal(tH.cpu().numpy(), wH)
            and np.array_equal(ema.cpu().numpy(), np.array(wst)),
            "tracked thresholds differ from the oracle's")
    stream = torch.cuda.current_stream()
    out = {}
    n = inp["x"].size
    for k, f in calls.items():
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        ts = np.array(ts)
        out[k] = {"us_median": round(float(np.median(ts)), 2), "us_min": round(float(ts.min()), 2),
                  "GB_s": round(5 * n / (np.median(ts) * 1e-6) / 1e9, 1)}
    out["softedge_over_int8"] = round(out["softedge"]["us_median"] / out["int8"]["us_median"], 3)
    out["track"]["GB_s"] = round(4 * 4 * n / (out["track"]["us_median"] * 1e-6) / 1e9, 1)
    out["workload"] = "mamba1-130m x: 8 x 1536 x 2048 fp32 -> codes, cluster gather, 8 groups"
    out["parity"] = ("codes of the three encoders bit-exact against the oracle; tracked "
                     "thresholds and EMA state equal to the oracle's")
    out["note"] = ("GB_s counts 5 bytes per value for the encoders and 4 reads of x for the "
                   "tracker (plus a state copy of 128 bytes)")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-configs", dest="all_configs", action="store_true", default=True,
                    help="also run the other configurations (default)")
    ap.add_argument("--only", dest="all_configs", action="store_false",
                    help="run the selected workload only")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (reference for the traffic counters)")
    ap.add_argument("--print-digest", action="store_true",
                    help="print the kernel-source digest of the workload and exit")
    args = ap.parse_args()
    if args.print_digest:
        print(sources_digest(args.workload))
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_state_space_amd as qs
    qs.load()
    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(torch, dev)
        return
    try:
        wl, res = run_workload(torch, dev, args.workload, args.steps, args.warmup, 10.0,
                               not args.no_cpu_baseline)
        out = {"metric": METRIC, "value": res["value"], "unit": "state-updates/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
               "data": "synthetic", "config": wl.config, "roofline": res["roofline"],
               "parity": res["parity"], "hbm_frac_dominant": res["hbm_frac_dominant"],
               "timing": "value: wall clock over the timed steps; roofline: HIP events on the "
                         "launch stream around every 2nd timed call of the dominant entry point "
                         "(mean; median and min also given)"}
        if "cpu_baseline" in res:
            out["cpu_baseline"] = res["cpu_baseline"]
        if "mfma" in res:
            out["mfma"] = res["mfma"]
        del wl
        if args.all_configs:
            others = {}
            for name in OTHERS:
                if name == args.workload:
                    continue
                w2, r2 = run_workload(torch, dev, name, min(args.steps, 30), min(args.warmup, 3),
                                      2.0, not args.no_cpu_baseline)
                e = {"workload": w2.config["workload"], "value": r2["value"],
                     "unit": "int8 ops/s" if w2.bound == "mfma" else "state-updates/s",
                     "ms_per_step": r2["ms_per_step"], "parity": r2["parity"],
                     "roofline": {k: r2["roofline"][k] for k in
                                  ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                   "kernel_us", "kernel_us_median", "kernel_us_min")}}
                if "cpu_baseline" in r2:
                    e["cpu_baseline"] = r2["cpu_baseline"]
                if "mfma" in r2:
                    e["mfma"] = r2["mfma"]
                others[name] = e
                del w2
                torch.cuda.empty_cache()
                print(f"[bench] {name}: {r2['ms_per_step']:.4f} ms/step", file=sys.stderr,
                      flush=True)
            others["quantizers"] = quantizer_row(torch, dev)
            print("[bench] quantizers done", file=sys.stderr, flush=True)
            others["instruction_rates"] = probe_row(torch, dev)
            out["other_configs"] = others
    except ParityError as e:
        print(json.dumps({"error": "parity gate failed", "detail": str(e)}), file=sys.stderr,
              flush=True)
        sys.exit(3)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
