"""The allocation-free scan entry point (qssm_scan_w8a8_noalloc, through the C-ABI) against the
workspace entry point qssm_scan_w8a8 on the same inputs: both run the same kernels, so y and h_last
must agree bit for bit. Two calls in a row on one GPU, the second with a smaller input (its staging
overwrites only part of what the first left in the library's array), then a request above the
array's size, which must be refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import qssm_synth as synth

pytestmark = pytest.mark.gpu


def run_both(dev, inp, G, gs, **kw):
    import torch
    import quantized_state_space_amd as qs
    import quantized_state_space_amd.workloads as wl
    lay = wl.Mamba1Layer(inp, G, gs, dev, **kw)
    lay.quantize()
    lay.scan()
    torch.cuda.synchronize()
    y_ws, h_ws = lay.y.clone(), lay.h_last.clone()
    if lay.y.dtype.is_floating_point:
        lay.y.fill_(float("nan"))
    else:
        lay.y.fill_(-77)
    lay.h_last.fill_(float("nan"))
    qs.qssm_scan_w8a8_noalloc(lay.args)
    torch.cuda.synchronize()
    assert torch.equal(lay.y, y_ws), "y differs between the two entry points"
    assert torch.equal(lay.h_last, h_ws), "h_last differs between the two entry points"
    return lay


def test_noalloc_two_calls_second_smaller(dev):
    print("\n[no-alloc scan: B=4 L=2048 D=512 N=16, then B=1 L=300 D=128 N=16]", flush=True)
    big = synth.mamba1_inputs(cfg=61, batch=4, seqlen=2048, dim=512, dstate=16,
                              x_dist="student_t", calib_batch=1)
    run_both(dev, big, 8, 4)
    small = synth.mamba1_inputs(cfg=62, batch=1, seqlen=300, dim=128, dstate=16, calib_batch=1,
                                with_h0=True)
    run_both(dev, small, 2, 4, with_h0=True)


def test_noalloc_other_forms(dev):
    """N = 64 (eight waves), fp32 staging (gs = 2 below the states per wave), soft-edge x, and an
    int8 output, each checked against the workspace entry point."""
    import quantized_state_space_amd as qs
    print("\n[no-alloc scan: N=64, fp32 staging, soft-edge x, int8 y]", flush=True)
    inp = synth.mamba1_inputs(cfg=63, batch=2, seqlen=333, dim=192, dstate=64, calib_batch=1)
    run_both(dev, inp, 3, 16)
    inp = synth.mamba1_inputs(cfg=64, batch=2, seqlen=130, dim=64, dstate=16, calib_batch=1)
    run_both(dev, inp, 2, 2)
    run_both(dev, inp, 2, 4, x_code=qs.QSSM_X_SOFTEDGE)
    D = inp["x"].shape[1]
    yg = (np.arange(D) % 3).astype(np.uint8)
    ys = np.float32([0.05, 0.08, 0.11])
    yb = np.linspace(-0.01, 0.01, D).astype(np.float32)
    run_both(dev, inp, 2, 4, y_out=(yg, ys, yb))


def test_noalloc_refuses_oversized_staging(dev):
    """Staging of B * Gbc * N * (L + 64) * 8 bytes above QSSM_SCAN_SCRATCH_BYTES is refused on the
    host (no launch: the argument block points at nothing)."""
    import quantized_state_space_amd as qs
    lib = qs.load()
    dummy = ctypes.c_void_p(4096)
    a = qs.ScanArgs(batch=64, seqlen=1024, dim=64, dstate=64, x_code=0, x_groups=1, x=dummy,
                    x_group_of=dummy, x_scales=dummy, delta=dummy, A=dummy, bc_groups=1,
                    bc_group_size=8, Bq=dummy, Cq=dummy, B_scales=dummy, C_scales=dummy, y=dummy,
                    y_dtype=0)
    assert 64 * 64 * (1024 + 64) * 8 > qs.QSSM_SCAN_SCRATCH_BYTES
    st = lib.qssm_scan_w8a8_noalloc(ctypes.byref(a), None)
    assert st == qs.QSSM_ERR_UNSUPPORTED
    assert b"scratch" in lib.qssm_last_error()
