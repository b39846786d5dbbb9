"""GPU parity of the SSD layer's int8 intra-chunk output (each row of the intra-chunk weights
W[i, j] = (C_i . B_j) exp(cum_i - cum_j) delta_j requantized with its own max / 127 scale, int8
MFMA against the x codes) against the oracle's mode of the same definition.

The requantized codes are floating-point decisions: the kernel forms W from G carried in fp16
(relative rounding 2^-11) and fp32 decay factors, and its row scale from that W, so a code t = W *
127 / m can differ from the oracle's by one step only where t lies within
    eps(t) = 1.2e-3 |t| + 1e-4
of a rounding boundary (2^-11 for G, the same for the row maximum, 1e-5 for the decay factors
and roundings, with margin). Each output is held to the fp32-state tolerance of its row plus,
for every such near-boundary code of its row, one requantization step times |xh_j[p]|. The
state is computed as without the option and must match as tightly as ever."""
import numpy as np
import pytest

import oracle
import oracle.pipelines as op
import qssm_synth as synth
from tests.test_gpu_ssd import TOL, check, run_layer, y_rows

pytestmark = pytest.mark.gpu

EPS_REL, EPS_ABS = 1.2e-3, 1e-4


def flip_allowance(inp, ref):
    out, near, total = op.ssd_intra_near_boundary(inp, ref, EPS_REL, EPS_ABS)
    print(f"  near-boundary codes: {near} of {total}", flush=True)
    return out


def check_intra(lay, ref, inp, heads=None):
    y = lay.y.float().cpu().numpy()
    if heads is not None:
        y = y[:, :, heads]
    r = np.asarray(ref["y"], np.float64)
    rows_r = y_rows(r)
    rowmax = np.abs(rows_r).max(axis=1, keepdims=True)
    allow = TOL * rowmax + y_rows(flip_allowance(inp, ref))
    err = np.abs(y_rows(y) - rows_r)
    slack_used = np.max(err / allow)
    print(f"  worst error / allowance {slack_used:.3f}, plain row error "
          f"{oracle.rowwise_error(y_rows(y), rows_r).max():.2e}", flush=True)
    assert np.all(err <= allow), slack_used


@pytest.mark.parametrize("L,with_h0", [(600, True), (256, False), (77, True)])
def test_ssd_int8_intra(dev, L, with_h0):
    import quantized_state_space_amd as qs
    print(f"\n[ssd int8 intra L={L} h0={with_h0}]", flush=True)
    inp = synth.ssd_inputs(cfg=42, batch=2, seqlen=L, nheads=4, headdim=64, dstate=128, ngroups=2,
                           calib_len=256, with_h0=with_h0)
    lay = run_layer(dev, inp, with_h0=with_h0, intra_mma=qs.QSSM_MMA_I8)
    ref = op.ssd(inp, with_h0=with_h0, int8_intra=True)
    # codes and the state exactly as without the option
    check(lay, ref, tol=np.inf)
    check_intra(lay, ref, inp)


def test_ssd_int8_intra_with_int8_state(dev):
    """Both int8 options together: against the oracle with both modes."""
    import quantized_state_space_amd as qs
    print("\n[ssd int8 intra + int8 state]", flush=True)
    inp = synth.ssd_inputs(cfg=43, batch=1, seqlen=520, nheads=4, headdim=64, dstate=128,
                           ngroups=2, calib_len=256, with_h0=True)
    lay = run_layer(dev, inp, with_h0=True, intra_mma=qs.QSSM_MMA_I8, state_mma=qs.QSSM_MMA_I8)
    ref = op.ssd(inp, with_h0=True, int8_intra=True, int8_state=True)
    check(lay, ref, tol=np.inf)
    check_intra(lay, ref, inp)


def test_ssd_int8_intra_exact_special_case(dev):
    """A = 0, delta = 1, C one-hot on state 0 and B codes with 127 at each chunk start: every
    requantized weight equals W, so the int8 output matches the fp16 product's definition to the
    usual tolerance (no near-boundary allowance needed: all t are integers)."""
    import quantized_state_space_amd as qs
    print("\n[ssd int8 intra special case]", flush=True)
    inp = synth.ssd_inputs(cfg=44, batch=1, seqlen=512, nheads=2, headdim=64, dstate=128,
                           ngroups=1, calib_len=256)
    r = synth.rng(44, 9)
    inp["A"] = np.zeros_like(inp["A"])
    inp["delta"] = np.ones_like(inp["delta"])
    Cv = np.zeros_like(inp["C"])
    Cv[..., 0] = 1.0
    Bv = np.zeros_like(inp["B"])
    Bv[..., 0] = r.integers(-127, 128, Bv.shape[:3])
    Bv[:, ::256, :, 0] = 127.0
    inp["B"], inp["C"] = Bv.astype(np.float32), Cv.astype(np.float32)
    inp["B_cal"], inp["C_cal"] = inp["B"][:1].copy(), inp["C"][:1].copy()
    lay = run_layer(dev, inp, intra_mma=qs.QSSM_MMA_I8)
    ref_i8 = op.ssd(inp, int8_intra=True)
    ref = op.ssd(inp)
    np.testing.assert_allclose(ref_i8["y"], ref["y"], rtol=1e-10, atol=1e-9)
    check(lay, ref)


def test_c4_int8_intra_full_size_sampled(dev):
    """Mamba2-8B-shaped layer with the int8 intra-chunk output: two sampled heads against the
    oracle, codes and state as without the option."""
    import quantized_state_space_amd as qs
    print("\n[c4 int8 intra full size]", flush=True)
    inp = synth.ssd_inputs(cfg=4, calib_len=256)
    heads = np.array([5, 77])
    lay = run_layer(dev, inp, intra_mma=qs.QSSM_MMA_I8)
    ref = op.ssd(inp, heads=heads, int8_intra=True)
    check(lay, ref, heads=heads, tol=np.inf)
    check_intra(lay, ref, inp, heads=heads)
