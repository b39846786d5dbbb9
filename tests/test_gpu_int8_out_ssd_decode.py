"""GPU parity of the persistent int8 output (the SSDi8 abstract: y + a per-channel correction term,
quantized with static per-group scales for the next W8A8 module) of the Mamba2 SSD layer and of the
decode update.

Two checks, as for the Mamba1 scan's int8 output:
- against the oracle's requantization of its fp64 y: the kernel's y is held to the fp32-state
  tolerance per row (2e-3 of the row's largest |y|), so a code may differ by one where v / s lies
  within that much (in code units) of a rounding boundary; every other code must be equal, none may
  differ by more than one;
- against the library's exact quantizer applied to fl32(y_f32 + bias) of the same layer run with an
  fp32 output: bit for bit (both runs compute the same fp32 y)."""
import numpy as np
import pytest

import oracle
import oracle.pipelines as op
import qssm_synth as synth
from tests.test_gpu_scan_int8_out import y_calib

pytestmark = pytest.mark.gpu

TOL = 2e-3


def check_codes_vs_oracle(got, y64, group_of, scales, bias, tol=TOL):
    """got, y64: [outer, C, inner]; rows are (outer, channel) over inner... the SSD and decode
    layouts put the channel last, so callers pass [outer, C, 1] views and row maxima per channel."""
    want = oracle.requant_output(y64, group_of, scales, bias)
    y32 = np.asarray(y64, np.float64).astype(np.float32)
    v = (y32 + bias[None, :, None]).astype(np.float32).astype(np.float64)
    s = np.asarray(scales, np.float64)[np.asarray(group_of, np.int64)][None, :, None]
    # per channel: tol x the channel's largest |y| over the whole run, in code units
    rowmax = np.abs(np.asarray(y64, np.float64)).max(axis=(0, 2), keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = v / s
        allow = tol * rowmax / s + 1e-6
        near = np.abs(r - np.floor(r) - 0.5) < allow
    diff = got.astype(np.int32) - want.astype(np.int32)
    far_bad = np.count_nonzero(diff[~near])
    print(f"  codes: {got.size} checked, {np.count_nonzero(near)} near a boundary, "
          f"{np.count_nonzero(diff)} differ", flush=True)
    assert far_bad == 0, f"{far_bad} codes away from a rounding boundary differ"
    assert np.abs(diff).max(initial=0) <= 1
    return int(np.count_nonzero(diff))


def consistency(dev, got_i8, y_f32, yg, ys, yb):
    """The int8 codes equal the library quantizer over fl32(y_f32 + bias) ([outer, C] views)."""
    import torch
    import quantized_state_space_amd as qs
    yb_t, yg_t, ys_t = (torch.from_numpy(a).to(dev) for a in (yb, yg, ys))
    v = (y_f32 + yb_t[None, :]).contiguous()
    want = torch.empty(v.shape, dtype=torch.int8, device=dev)
    qs.qssm_quant_group_x(v.view(v.shape[0], v.shape[1], 1), yg_t, int(ys.size), ys_t,
                          want.view(v.shape[0], v.shape[1], 1))
    torch.cuda.synchronize()
    assert torch.equal(got_i8, want)


@pytest.mark.parametrize("L,with_h0,Gy,spread", [(600, True, 4, (1.0, 0.5)), (300, False, 1, (1.0,)),
                                                 (77, True, 3, (0.4, 1.0, 1.0))])
def test_ssd_int8_output(dev, L, with_h0, Gy, spread):
    import torch
    import quantized_state_space_amd.workloads as wl
    print(f"\n[ssd int8 y L={L} h0={with_h0} Gy={Gy}]", flush=True)
    inp = synth.ssd_inputs(cfg=51, batch=2, seqlen=L, nheads=4, headdim=64, dstate=128, ngroups=2,
                           calib_len=256, with_h0=with_h0)
    ref = op.ssd(inp, with_h0=with_h0)
    B, _, nh, P = inp["x"].shape
    y64 = np.asarray(ref["y"], np.float64).reshape(B * L, nh * P, 1)
    yg, ys, yb = y_calib(y64, Gy, 51, spread)
    lay_q = wl.SsdLayer(inp, dev, with_h0=with_h0, y_out=(yg, ys, yb))
    lay_f = wl.SsdLayer(inp, dev, with_h0=with_h0)
    lay_q.step()
    lay_f.step()
    torch.cuda.synchronize()
    assert lay_q.y.dtype == torch.int8
    got = lay_q.y.cpu().numpy().reshape(B * L, nh * P, 1)
    check_codes_vs_oracle(got, y64, yg, ys, yb)
    consistency(dev, lay_q.y.view(B * L, nh * P), lay_f.y.view(B * L, nh * P), yg, ys, yb)
    # the state is the same as with an fp32 output
    assert torch.equal(lay_q.h_last, lay_f.h_last)


def test_ssd_int8_output_invalid_scale_no_bias(dev):
    import torch
    import quantized_state_space_amd.workloads as wl
    print("\n[ssd int8 y invalid scale, no bias]", flush=True)
    inp = synth.ssd_inputs(cfg=52, batch=1, seqlen=256, nheads=2, headdim=64, dstate=128, ngroups=1,
                           calib_len=256)
    ref = op.ssd(inp)
    y64 = np.asarray(ref["y"], np.float64).reshape(256, 128, 1)
    yg, ys, _ = y_calib(y64, 3, 52)
    ys = ys.copy()
    ys[1] = np.float32(2.0 ** 101)
    lay = wl.SsdLayer(inp, dev, y_out=(yg, ys, None))
    lay.step()
    torch.cuda.synchronize()
    got = lay.y.cpu().numpy().reshape(256, 128, 1)
    assert not got[:, yg == 1].any()
    check_codes_vs_oracle(got, y64, yg, ys, np.zeros(128, np.float32))


def test_c4_int8_output_full_size(dev):
    """Mamba2-8B-shaped layer with an int8 output in 8 groups per head block, as the benchmark's
    int8-output SSD workload runs it: the codes equal the library quantizer over the fp32 run bit
    for bit, and two sampled heads match the oracle."""
    import torch
    import quantized_state_space_amd.workloads as wl
    print("\n[c4 int8 y full size]", flush=True)
    inp = synth.ssd_inputs(cfg=4, calib_len=256)
    heads = np.array([3, 100])
    ref = op.ssd(inp, heads=heads)
    B, L, nh, P = inp["x"].shape
    C = nh * P
    yg = (np.arange(C) * 64 // C).astype(np.uint8)
    top = np.float32(np.abs(ref["y"]).max())
    ys = oracle.scale_from_absmax(np.full(64, top * np.float32(0.7), np.float32))
    yb = (synth.rng(53, 12).standard_normal(C) * 0.01 * top).astype(np.float32)
    lay_q = wl.SsdLayer(inp, dev, y_out=(yg, ys, yb))
    lay_q.step()
    torch.cuda.synchronize()
    qy = lay_q.y.clone()
    del lay_q
    torch.cuda.empty_cache()
    lay_f = wl.SsdLayer(inp, dev)
    lay_f.step()
    consistency(dev, qy.view(B * L, C), lay_f.y.view(B * L, C), yg, ys, yb)
    ch = (heads[:, None] * P + np.arange(P)[None, :]).reshape(-1)
    got = qy.cpu().numpy()[:, :, heads].reshape(B * L, len(ch), 1)
    check_codes_vs_oracle(got, np.asarray(ref["y"], np.float64).reshape(B * L, len(ch), 1),
                          yg[ch], ys, yb[ch])


@pytest.mark.parametrize("state", ["f32", "f16"])
def test_decode_int8_output(dev, state):
    """Decode with an int8 output over 5 tokens: every token's codes against the oracle (tolerance
    of the state type) and bit for bit against the library quantizer over an fp32-output run."""
    import torch
    import quantized_state_space_amd as qs
    import quantized_state_space_amd.workloads as wl
    print(f"\n[decode int8 y {state}]", flush=True)
    dims = dict(batch=6, nheads=16, headdim=64, dstate=128, ngroups=2)
    params = synth.decode_params(cfg=54, **dims)
    steps = [synth.decode_step_inputs(k, cfg=54, **dims) for k in range(5)]
    sd = qs.QSSM_F32 if state == "f32" else qs.QSSM_F16
    tol = 2e-3 if state == "f32" else 1e-2
    if sd == qs.QSSM_F16:
        params["state0"] = params["state0"].astype(np.float16).astype(np.float32)
    ref = op.decode(params, steps)
    C = 16 * 64
    y64 = np.stack([np.asarray(y, np.float64).reshape(6, C) for y in ref["y"]])   # [T, B, C]
    yg, ys, yb = y_calib(y64.reshape(-1, C, 1), 4, 54, (1.0, 0.6))
    lay_q = wl.DecodeLayer(params, dev, state_dtype=sd, y_out=(yg, ys, yb))
    lay_f = wl.DecodeLayer(params, dev, state_dtype=sd)
    for k, inp in enumerate(steps):
        for lay in (lay_q, lay_f):
            lay.load_inputs(inp)
            lay.step()
        torch.cuda.synchronize()
        got = lay_q.y.cpu().numpy().reshape(6, C, 1)
        check_codes_vs_oracle(got, y64[k].reshape(6, C, 1), yg, ys, yb, tol=tol)
        consistency(dev, lay_q.y.view(6, C), lay_f.y.view(6, C), yg, ys, yb)
