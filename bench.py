"""Benchmark of the quantized state-space hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3|c3se|c3i8y|c1|c2|c4|c4f16|c5|c5f16]
                [--only] [--no-cpu-baseline]

One step = one pass of the whole hot path of the workload over one batch of synthetic input that is
already resident in HBM: for the Mamba1 layers, quantize x (gathered into cluster order), quantize B
and C, run the W8A8 scan; for S4D, quantize the input then scan; for the SSD layer, quantize x, B, C
then run the chunked SSD; for decode, one fused state update of every sequence.

Prints one JSON line: throughput in state-updates/s (B*L*D*N per step), the dominant kernel's
roofline figures measured with HIP events on the launch stream, and the oracle timed on this host.
Unless --only is given, the line also carries a short run of the other configurations
(other_configs: S4D, soft-edge Mamba1, SSD, decode fp32 and fp16) with their own rooflines.
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
# fp32 VALU issue rate of MI355X without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# (lane-instructions per second; an FMA counts once). The recurrences' instruction mix (an exp per
# update, dependent FMAs) is compiled without packed fp32 instructions.
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
METRIC = "quantized scan state-updates/s (B·L·D·N) + % of HBM peak, 1 MI355X"


# ------------------------------------------------------------------------------------------------
# workloads

class Workload:
    name = ""
    dominant = ""           # kernel timed for the roofline
    bound = "hbm"
    config: dict = {}

    def setup(self, dev): ...
    def step(self, timer): ...
    def updates(self): ...
    def dominant_bytes(self): ...
    def cpu_baseline(self): ...


class Mamba1(Workload):
    # per state update: v_mul (delta * A log2 e), v_exp_f32, v_mul (delta x * B), two FMAs (state
    # and readout)
    ops_per_update = 5

    def __init__(self, soft_edge=False, y_int8=False):
        self.soft = soft_edge
        self.y_int8 = y_int8
        self.name = ("mamba1-130m-layer-w8a8" + ("-softedge-x" if soft_edge else "") +
                     ("-int8-y" if y_int8 else ""))
        self.dominant = "qssm_scan_w8a8: k_stage_bc + k_scan_m1"
        self.bound = "alu"

    def setup(self, dev):
        import qssm_synth as synth
        import quantized_state_space_amd as qs
        import quantized_state_space_amd.workloads as wl
        self.inp = synth.c3_inputs()
        xc = qs.QSSM_X_SOFTEDGE if self.soft else qs.QSSM_X_INT8
        # two copies of every buffer, used in turn, so that one step's 350 MB of traffic cannot be
        # served from the previous step's lines in the 256 MB last-level cache
        y_out = None
        if self.y_int8:
            # int8 output for the next W8A8 module: 8 clustered output groups calibrated on one
            # fp32-output pass, and a seeded per-channel correction term (~1% of a channel's range)
            import numpy as np
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
        self.layers = [wl.Mamba1Layer(self.inp, 8, 4, dev, x_code=xc, y_out=y_out)
                       for _ in range(2)]
        self.k = 0
        B, D, L, N, Gbc = self.layers[0].shape
        self.dims = (B, D, L, N, Gbc)
        self.config = {"workload": self.name, "batch": B, "seqlen": L, "d_inner": D, "d_state": N,
                       "x_groups": 8, "x_code": "soft-edge 3-scale u8" if self.soft else "int8",
                       "bc_state_groups": N // 4, "state": "f32",
                       "y": "int8, 8 output groups + per-channel correction" if self.y_int8
                       else "f32"}

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

    def cpu_baseline(self):
        import oracle.pipelines as op
        cal = op.mamba1_calib(self.inp, 8, 4, soft_edge=self.soft)
        reps, dt = timed_reps(lambda: op.mamba1(self.inp, G=8, gs=4, soft_edge=self.soft, calib=cal))
        return reps * self.updates() / dt, f"full workload (8 x 1536 channels x 2048 steps) x {reps}: " \
            "quantize, dequantize, fp64 scan"


class Tiny(Mamba1):
    def __init__(self):
        self.soft = False
        self.name = "tiny-mamba1-w8a8"
        self.dominant = "qssm_scan_w8a8: k_stage_bc + k_scan_m1"
        self.bound = "alu"

    def setup(self, dev):
        import qssm_synth as synth
        import quantized_state_space_amd.workloads as wl
        self.inp = synth.c1_inputs()
        self.layers = [wl.Mamba1Layer(self.inp, 1, 4, dev, dynamic_scales=True)]
        self.k = 0
        self.dims = self.layers[0].shape
        B, D, L, N, _ = self.dims
        self.config = {"workload": self.name, "batch": B, "seqlen": L, "d_inner": D, "d_state": N,
                       "x_groups": 1, "bc_state_groups": 4, "state": "f32", "y": "f32"}

    def cpu_baseline(self):
        import oracle.pipelines as op
        reps, dt = timed_reps(lambda: op.mamba1(self.inp, G=1, gs=4, dynamic=True))
        return reps * self.updates() / dt, f"full workload x {reps}"


class S4d(Workload):
    def __init__(self, i16=False):
        self.i16 = i16
        self.name = "s4d-smnist-shaped" + ("-int16-state" if i16 else "")
        self.dominant = "qssm_s4d_scan: k_s4d"
        self.bound = "alu"

    def setup(self, dev):
        import qssm_synth as synth
        import quantized_state_space_amd as qs
        import quantized_state_space_amd.workloads as wl
        self.inp = synth.s4d_inputs()
        ss = None
        self.lay = wl.S4dLayer(self.inp, dev, state_dtype=qs.QSSM_I16 if self.i16 else qs.QSSM_F32,
                               state_scale=ss)
        self.ss = ss
        B, L, H, N = self.lay.shape
        self.dims = (B, L, H, N)
        self.config = {"workload": self.name, "batch": B, "seqlen": L, "channels": H,
                       "d_state_complex": N, "state": "int16" if self.i16 else "f32", "y": "f32"}

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

    def dominant_bytes(self):
        B, L, H, N = self.dims
        return B * L + H + 6 * H * N + 4 * 8 * H + 4 * B * H * L + 8 * B * H * N

    # per complex state update, in the cheapest form the kernel uses (the chain on g = h / Bbar'):
    # Abar g + q (4 FMA-class) and Re(C' g) (2 FMA-class)
    ops_per_update = 6

    def ops(self):
        return self.ops_per_update * self.updates()

    def cpu_baseline(self):
        import oracle.pipelines as op
        reps, dt = timed_reps(lambda: op.s4d(self.inp, state_scale=self.ss))
        return reps * self.updates() / dt, f"full workload x {reps}, fp64 complex scan"


class Decode(Workload):
    def __init__(self, f16=False):
        self.f16 = f16
        self.name = "mamba2-8b-decode" + ("-fp16-state" if f16 else "")
        self.dominant = "qssm_state_update: k_state_update"

    def setup(self, dev):
        import torch
        import qssm_synth as synth
        import quantized_state_space_amd as qs
        import quantized_state_space_amd.workloads as wl
        self.params = synth.decode_params()
        self.lay = wl.DecodeLayer(self.params, dev, state_dtype=qs.QSSM_F16 if self.f16 else qs.QSSM_F32)
        B, nh, P, N, Gbc = self.lay.shape
        self.dims = self.lay.shape
        self.nsteps = 64
        self.inputs = [synth.decode_step_inputs(k) for k in range(self.nsteps)]
        # all 64 tokens resident in HBM; one argument block per token
        self.dev_inputs = []
        self.args = []
        for k, inp in enumerate(self.inputs):
            d = {n: torch.from_numpy(inp[n]).to(dev) for n in ("x", "B", "C", "delta")}
            self.dev_inputs.append(d)
            self.args.append(qs.update_args(d["x"], self.lay.group_t, self.lay.xs, d["B"], d["C"],
                                            self.lay.bs, self.lay.cs, 16, d["delta"], self.lay.A,
                                            self.lay.state, self.lay.y, Dskip=self.lay.D))
        self.k = 0
        self.config = {"workload": self.name, "batch": B, "heads": nh, "headdim": P, "d_state": N,
                       "ngroups": Gbc, "tokens": self.nsteps, "state": "f16" if self.f16 else "f32"}

    def step(self, timer):
        import quantized_state_space_amd as qs
        timer.start()
        qs.qssm_state_update(self.args[self.k % self.nsteps])
        timer.stop()
        self.k += 1

    def updates(self):
        B, nh, P, N, _ = self.dims
        return B * nh * P * N

    def dominant_bytes(self):
        B, nh, P, N, Gbc = self.dims
        sb = 2 if self.f16 else 4
        return 2 * sb * B * nh * P * N + 4 * (2 * B * nh * P + 2 * B * Gbc * N + B * nh)

    def cpu_baseline(self):
        import oracle.pipelines as op
        sample = np.arange(16)
        reps, dt = timed_reps(lambda: op.decode(self.params, self.inputs[:8], batches=sample))
        B, nh, P, N, _ = self.dims
        return reps * 8 * len(sample) * nh * P * N / dt, \
            f"16 of 256 sequences x 8 tokens (fp64 state) x {reps}"


class Ssd(Workload):
    def __init__(self, f16=False):
        self.f16 = f16
        self.name = "mamba2-8b-ssd-layer-w8a8" + ("-fp16-y" if f16 else "")
        self.dominant = "qssm_ssd_chunk_int8: k_ssd_state + k_ssd_output"

    def setup(self, dev):
        import qssm_synth as synth
        import quantized_state_space_amd as qs
        import quantized_state_space_amd.workloads as wl
        self.inp = synth.ssd_inputs(cfg=4, calib_len=256)
        self.lay = wl.SsdLayer(self.inp, dev, y_dtype=qs.QSSM_F16 if self.f16 else qs.QSSM_F32)
        B, L, nh, P, N, Gbc = self.lay.shape
        self.dims = self.lay.shape
        self.config = {"workload": self.name, "batch": B, "seqlen": L, "heads": nh, "headdim": P,
                       "d_state": N, "ngroups": Gbc, "chunk": 256, "x_groups": int(self.lay.G),
                       "bc_state_groups": N // 16, "state": "f32", "y": "f16" if self.f16 else "f32"}

    def step(self, timer):
        self.lay.quantize()
        timer.start()
        self.lay.scan()
        timer.stop()

    def updates(self):
        B, L, nh, P, N, _ = self.dims
        return B * L * nh * P * N

    def dominant_bytes(self):
        B, L, nh, P, N, Gbc = self.dims
        yb = 2 if self.f16 else 4
        # x codes, delta, B/C codes, A, D in; y out; h_last out (each once)
        return B * L * nh * P * (1 + yb) + 4 * B * L * nh + 2 * B * L * Gbc * N + 8 * nh + \
            4 * B * nh * P * N

    def cpu_baseline(self):
        import oracle.pipelines as op
        heads = np.array([0, 64])
        reps, dt = timed_reps(lambda: op.ssd(self.inp, heads=heads))
        B, L, nh, P, N, _ = self.dims
        return reps * B * L * len(heads) * P * N / dt, f"2 of 128 heads (all batches, full " \
            f"length) x {reps}: fp64 chunked form incl. quantizing the layer's x, B, C"


_zc = {}


def timed_reps(fn, min_seconds=10.0):
    """Runs fn until at least min_seconds of wall time have passed; returns (reps, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return reps, dt


def _zero(device):
    import torch
    k = str(device)
    if k not in _zc:
        _zc[k] = torch.zeros(1, dtype=torch.uint8, device=device)
    return _zc[k]


WORKLOADS = {"c3": lambda: Mamba1(False), "c3se": lambda: Mamba1(True),
             "c3i8y": lambda: Mamba1(False, True), "c1": Tiny,
             "c2": lambda: S4d(False), "c4": lambda: Ssd(False), "c4f16": lambda: Ssd(True),
             "c5": lambda: Decode(False),
             "c5f16": lambda: Decode(True)}


# ------------------------------------------------------------------------------------------------

# HBM traffic of one call of the dominant entry point, from two rocprofv3 counter runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, summed over the call's kernels), each divided by
# the ratio the same counter reads for a plain 1 GiB device copy (bench.py --copy-probe). Keyed by
# workload: (fetch bytes, write bytes, sha256 of the kernel sources when the counters were taken).
TRAFFIC = {
    "c3": (152089444, 132508472, "82855a741382f2d7"),
    "c2": (374806, 7472096, "a1d2ef04c9625eb6"),
    "c4": (692105038, 858799064, "1771bfe3189ad294"),
    "c5": (1100171354, 1082578296, "2d61ee22651a7256"),
    "c3se": (152357308, 132879688, "82855a741382f2d7"),
    "c3i8y": (135567360, 27820032, "82855a741382f2d7"),
    "c4f16": (683357980, 694246608, "1771bfe3189ad294"),
    "c5f16": (563235239, 545288304, "2d61ee22651a7256"),
}
TRAFFIC_SOURCES = {
    "c1": ["scan_m1.hip"], "c3": ["scan_m1.hip"], "c3se": ["scan_m1.hip"],
    "c3i8y": ["scan_m1.hip"], "c2": ["s4d.hip"],
    "c4": ["ssd.hip"], "c4f16": ["ssd.hip"], "c5": ["state_update.hip"],
    "c5f16": ["state_update.hip"],
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
    every `every`-th timed call (a pair of event records costs ~6 us of stream time per call, which
    would otherwise be charged to the step)."""

    def __init__(self, torch, every=4):
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

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs]))


def run_workload(torch, dev, name, steps, warmup):
    """Sets up workload `name`, runs warmup + timed steps; returns (workload, results)."""
    wl = WORKLOADS[name]()
    wl.setup(dev)
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
    kern_ms = timer.mean_ms()
    nbytes = wl.dominant_bytes()
    if wl.bound == "alu":
        achieved = wl.ops() / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(achieved, 3), "peak": round(VALU_PEAK_TOPS, 2),
                "unit": "T VALU lane-ops/s", "frac": round(achieved / VALU_PEAK_TOPS, 4)}
    else:
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(name)
    roof["kernel"] = wl.dominant
    roof["kernel_us"] = round(kern_ms * 1e3, 2)
    roof["algorithmic_bytes"] = int(nbytes)
    if wl.bound == "alu":
        roof["ops_per_update"] = wl.ops_per_update
    res = {"value": wl.updates() * steps / elapsed, "ms_per_step": elapsed * 1e3 / steps,
           "roofline": roof,
           "hbm_frac_dominant": round(nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return wl, res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-configs", dest="all_configs", action="store_true", default=True,
                    help="also run the other configurations briefly (default)")
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
    wl, res = run_workload(torch, dev, args.workload, args.steps, args.warmup)
    out = {"metric": METRIC, "value": res["value"], "unit": "state-updates/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic", "config": wl.config, "roofline": res["roofline"],
           "hbm_frac_dominant": res["hbm_frac_dominant"],
           "timing": "HIP events on the launch stream around every 4th timed call of the "
                     "dominant entry point; value from the wall clock over the timed steps"}
    if not args.no_cpu_baseline:
        v, sample = wl.cpu_baseline()
        import oracle
        threads = oracle.max_threads()
        out["cpu_baseline"] = {"value": v, "unit": "state-updates/s", "cores": threads,
                               "kind": "oracle", "sample": sample}
    del wl
    if args.all_configs:
        # the other configurations of the same metric, briefly (same protocol, fewer steps)
        others = {}
        for name in ("c2", "c3se", "c3i8y", "c4", "c5", "c5f16"):
            if name == args.workload:
                continue
            w2, r2 = run_workload(torch, dev, name, min(args.steps, 30), min(args.warmup, 3))
            others[name] = {"workload": w2.config["workload"], "value": r2["value"],
                            "ms_per_step": r2["ms_per_step"],
                            "roofline": {k: r2["roofline"][k] for k in
                                         ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                          "kernel_us")}}
            del w2
            torch.cuda.empty_cache()
        out["other_configs"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
