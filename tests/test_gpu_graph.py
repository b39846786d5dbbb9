"""The library under HIP graph capture: it allocates nothing, synchronizes nothing and records no
memset, so a layer step can be captured once and replayed. Each test captures a step, then replays
it several times on new inputs written into the same buffers by ordinary eager work (with a
synchronization before and after every replay), and checks every replay bit for bit against the
same step run eagerly on those inputs."""
import numpy as np
import pytest

import qssm_synth as synth

pytestmark = pytest.mark.gpu


def capture(torch, fn):
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_mamba1_layer_step_replays(dev):
    """Quantize x (with the cluster gather), quantize B and C, stage and scan: five kernels."""
    import torch
    import quantized_state_space_amd.workloads as wl
    print("\n[graph: mamba1 layer step]", flush=True)
    inp = synth.mamba1_inputs(cfg=21, batch=2, seqlen=300, dim=128, dstate=16, calib_batch=1)
    lay = wl.Mamba1Layer(inp, 4, 4, dev)
    ref = wl.Mamba1Layer(inp, 4, 4, dev)
    g = capture(torch, lay.step)
    r = np.random.default_rng(21)
    for k in range(3):
        x = torch.from_numpy(inp["x"] * np.float32(1 + 0.3 * k)).to(dev)
        B = torch.from_numpy(r.standard_normal(inp["B"].shape).astype(np.float32)).to(dev)
        C = torch.from_numpy(r.standard_normal(inp["C"].shape).astype(np.float32)).to(dev)
        for l in (lay, ref):
            l.x.copy_(x)
            l.Bf.copy_(B)
            l.Cf.copy_(C)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref.step()
        torch.cuda.synchronize()
        for name in ("xq", "Bq", "Cq", "y", "h_last"):
            assert torch.equal(getattr(lay, name), getattr(ref, name)), (k, name)


def test_ssd_layer_step_replays(dev):
    """Quantize x, B, C, then the two SSD kernels."""
    import torch
    import quantized_state_space_amd.workloads as wl
    print("\n[graph: ssd layer step]", flush=True)
    inp = synth.ssd_inputs(cfg=22, batch=1, seqlen=300, nheads=4, headdim=64, dstate=128,
                           ngroups=2, calib_len=256)
    lay = wl.SsdLayer(inp, dev)
    ref = wl.SsdLayer(inp, dev)
    g = capture(torch, lay.step)
    for k in range(3):
        x = torch.from_numpy(inp["x"] * np.float32(1 - 0.2 * k)).to(dev)
        for l in (lay, ref):
            l.x.copy_(x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref.step()
        torch.cuda.synchronize()
        for name in ("xq", "Bq", "Cq", "y", "h_last"):
            assert torch.equal(getattr(lay, name), getattr(ref, name)), (k, name)


def test_decode_steps_replay(dev):
    """The fused decode update, which changes the state in place: the captured step replayed on
    successive tokens follows the eager run token by token."""
    import torch
    import quantized_state_space_amd as qs
    import quantized_state_space_amd.workloads as wl
    print("\n[graph: decode steps]", flush=True)
    dims = dict(batch=4, nheads=8, headdim=64, dstate=128, ngroups=2)
    params = synth.decode_params(cfg=23, **dims)
    steps = [synth.decode_step_inputs(k, cfg=23, **dims) for k in range(4)]
    lay = wl.DecodeLayer(params, dev, state_dtype=qs.QSSM_F32, emit_codes=True)
    ref = wl.DecodeLayer(params, dev, state_dtype=qs.QSSM_F32, emit_codes=True)
    lay.load_inputs(steps[0])
    g = capture(torch, lay.step)
    lay.state.copy_(ref.state)  # the warm-up ran one real step: start both from the same state
    torch.cuda.synchronize()
    for k, s in enumerate(steps):
        lay.load_inputs(s)
        ref.load_inputs(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref.step()
        torch.cuda.synchronize()
        assert torch.equal(lay.y, ref.y), k
        assert torch.equal(lay.state, ref.state), k
        for a, b in zip(lay.codes, ref.codes):
            assert torch.equal(a, b), k
