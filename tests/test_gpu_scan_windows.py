"""GPU parity of the Mamba1 scan's time-window form (each window's end state from zero, carries
between windows, then the windows again from their entering states) against the oracle's
sequential fp64 scan: the same codes, y and h_last within the fp32-state tolerance per row, over
window counts, ragged lengths (a partial last window), state sizes (every kernel shape), soft-edge
x, fp16 y and h0; and the library's own choice at the tiny-layer size."""
import numpy as np
import pytest

import oracle
import oracle.pipelines as op
import qssm_synth as synth
from tests.test_gpu_scan import TOL_F32, assert_rows_close, check_codes, layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,D,L,N,K,soft,gs", [(2, 100, 300, 16, 2, False, 4),
                                                (1, 64, 77, 4, 3, False, 4),
                                                (2, 192, 520, 8, 16, False, 4),
                                                (1, 128, 200, 32, 5, True, 4),
                                                (1, 64, 129, 64, 9, False, 16),
                                                (1, 64, 1000, 16, 64, False, 2),   # -> 16
                                                (2, 70, 2048, 16, 7, True, 1)])
def test_windows_match_oracle(dev, B, D, L, N, K, soft, gs):
    import quantized_state_space_amd as qs
    print(f"\n[mamba1 windows B={B} D={D} L={L} N={N} K={K} softedge={soft} gs={gs}]", flush=True)
    inp = synth.mamba1_inputs(cfg=15, batch=B, seqlen=L, dim=D, dstate=N, x_dist="student_t",
                              calib_batch=1, with_h0=True)
    xc = qs.QSSM_X_SOFTEDGE if soft else qs.QSSM_X_INT8
    lay = layer(dev, inp, G=3, gs=gs, x_code=xc, with_h0=True, time_blocks=K)
    lay.step()
    ref = op.mamba1(inp, G=3, gs=gs, soft_edge=soft, with_h0=True)
    check_codes(lay, ref)
    assert_rows_close(lay.y.cpu().numpy(), ref["y"], TOL_F32)
    assert_rows_close(lay.h_last.cpu().numpy(), ref["h_last"], TOL_F32, "h_last")


def test_windows_fp16_output_and_chain_agreement(dev):
    """fp16 y through windows; and the windowed fp32 y agrees with the chain form's."""
    import torch
    import quantized_state_space_amd as qs
    print("\n[mamba1 windows fp16 y]", flush=True)
    inp = synth.mamba1_inputs(cfg=16, batch=2, seqlen=640, dim=128, dstate=16,
                              x_dist="student_t", calib_batch=1, with_h0=True)
    ref = op.mamba1(inp, G=4, gs=4, with_h0=True)
    lw = layer(dev, inp, G=4, gs=4, with_h0=True, time_blocks=10, y_dtype=qs.QSSM_F16)
    lw.step()
    torch.cuda.synchronize()
    assert lw.y.dtype == torch.float16
    assert_rows_close(lw.y.float().cpu().numpy(), ref["y"], TOL_F32)
    a = layer(dev, inp, G=4, gs=4, with_h0=True, time_blocks=10)
    c = layer(dev, inp, G=4, gs=4, with_h0=True, time_blocks=1)
    a.step()
    c.step()
    torch.cuda.synchronize()
    assert_rows_close(a.y.cpu().numpy(), c.y.cpu().numpy().astype(np.float64), TOL_F32)
    assert_rows_close(a.h_last.cpu().numpy(), c.h_last.cpu().numpy().astype(np.float64), TOL_F32)


def test_library_choice_at_tiny_size(dev):
    """The tiny Mamba1 layer (B=1, D=64, N=16, L=256, on-device scales) with the library's choice,
    which cuts it into time windows, against the oracle."""
    print("\n[c1 library choice]", flush=True)
    inp = synth.c1_inputs()
    lay = layer(dev, inp, G=1, gs=4, dynamic_scales=True)
    lay.step()
    ref = op.mamba1(inp, G=1, gs=4, dynamic=True)
    check_codes(lay, ref)
    assert_rows_close(lay.y.cpu().numpy(), ref["y"], TOL_F32)
    assert_rows_close(lay.h_last.cpu().numpy(), ref["h_last"], TOL_F32, "h_last")


def test_windows_without_h0_and_h_last(dev):
    """No h0 (windows start from zero throughout) and no h_last requested."""
    import torch
    import quantized_state_space_amd as qs
    import quantized_state_space_amd.workloads as wl
    print("\n[mamba1 windows, no h0 / h_last]", flush=True)
    inp = synth.mamba1_inputs(cfg=17, batch=1, seqlen=333, dim=64, dstate=16, x_dist="normal",
                              calib_batch=1)
    lay = wl.Mamba1Layer(inp, 2, 4, dev, time_blocks=4)
    lay.args.h_last = None
    lay.step()
    torch.cuda.synchronize()
    ref = op.mamba1(inp, G=2, gs=4)
    assert_rows_close(lay.y.cpu().numpy(), ref["y"], TOL_F32)
