"""GPU parity of the soft-edge variants (Quamba-SE blog, section 4.1) against the oracle:
- the shift-only form (scale/2, scale*2): encode and decode bit for bit;
- on-device threshold tracking (P5 / P99.9 of |x| per group, EMA over batches): s, L, H and the
  fp64 EMA state equal the oracle's bit for bit, over layouts, permutations, group counts, ties,
  tiny and empty groups, and a chain of batches;
- the Mamba1 scan on shift-only x, on soft-edge B/C (both forms, both staging layouts) and with
  tracked thresholds: codes bit-exact, y and h_last within the fp32-state tolerance per row."""
import numpy as np
import pytest

import oracle
import oracle.pipelines as op
import qssm_synth as synth
from tests.test_gpu_scan import TOL_F32, assert_rows_close

pytestmark = pytest.mark.gpu


def T(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("perm_on", [True, False])
def test_shift_form_encode_decode_bit_exact(dev, perm_on):
    import torch
    import quantized_state_space_amd as qs
    print(f"\n[softedge shift form perm={perm_on}]", flush=True)
    r = synth.rng(61, 0)
    outer, C, inner, G = 2, 96, 200, 3
    x = (r.standard_t(3, (outer, C, inner))).astype(np.float32)
    x.flat[::89] = np.nan
    x.flat[1::173] = np.inf
    x.flat[2::179] = -np.inf
    x.flat[3::181] = -0.0
    # values on the mode scales' rounding boundaries and next to them
    k = r.integers(-40, 40, 4000) + 0.5
    ties = (k * 0.05 / 2).astype(np.float32)
    x.flat[5:5 + ties.size * 3:3] = ties
    x.flat[6:6 + ties.size * 3:3] = np.nextafter(ties, np.float32(np.inf))
    group_of = r.integers(0, G, C).astype(np.uint8)
    perm = r.permutation(C).astype(np.int32) if perm_on else None
    s = np.array([0.05, 0.02, 0.3], np.float32)
    L = np.array([0.1, 0.0, 0.5], np.float32)
    H = np.array([3.0, 1.0, 0.2], np.float32)
    code = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    qs.qssm_softedge_encode(T(x, dev), T(group_of, dev), G, T(s, dev), T(L, dev), T(H, dev), code,
                            perm=None if perm is None else T(perm, dev), form=qs.QSSM_X_SOFTEDGE2)
    out = torch.empty(x.shape, dtype=torch.float32, device=dev)
    qs.qssm_softedge_decode(code, T(group_of, dev), G, T(s, dev), out, form=qs.QSSM_X_SOFTEDGE2)
    torch.cuda.synchronize()
    want = oracle.softedge_encode(x, group_of, s, L, H, perm=perm, ratio=2)
    assert np.array_equal(code.cpu().numpy(), want)
    dec = oracle.softedge_decode_f32(want, group_of, s, ratio=2)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), dec.view(np.uint32))


def test_shift_form_decode_all_bytes(dev):
    import torch
    import quantized_state_space_amd as qs
    scales = np.array([1.0, 0.0173, 2.0 ** -100, 2.0 ** 100, 0.0], np.float32)
    codes = np.tile(np.arange(256, dtype=np.uint8), (1, len(scales), 1))
    out = torch.empty(codes.shape, dtype=torch.float32, device=dev)
    qs.qssm_softedge_decode(T(codes, dev), T(np.arange(len(scales), dtype=np.uint8), dev),
                            len(scales), T(scales, dev), out, form=qs.QSSM_X_SOFTEDGE2)
    torch.cuda.synchronize()
    want = np.stack([oracle.softedge_value_table(s, 2).astype(np.float32) for s in scales])[None]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------------------------------------------
# on-device threshold tracking

def run_track(dev, x, group_of, G, perm=None, prev=None, alpha=0.1):
    import torch
    import quantized_state_space_amd as qs
    st = torch.zeros((G, 2), dtype=torch.float64, device=dev)
    if prev is not None:
        st.copy_(torch.from_numpy(np.asarray(prev, np.float64)))
    s = torch.empty(G, dtype=torch.float32, device=dev)
    L = torch.empty(G, dtype=torch.float32, device=dev)
    H = torch.empty(G, dtype=torch.float32, device=dev)
    ws = torch.empty(qs.qssm_softedge_track_workspace_size(G), dtype=torch.uint8, device=dev)
    ws.fill_(0xAB)   # the call must clear what it uses
    qs.qssm_softedge_track(T(x, dev), T(group_of, dev), G, st, s, L, H, ws,
                           ema_valid=prev is not None, perm=None if perm is None else T(perm, dev),
                           alpha=alpha)
    torch.cuda.synchronize()
    return s.cpu().numpy(), L.cpu().numpy(), H.cpu().numpy(), st.cpu().numpy()


def check_track(got, want):
    s, L, H, st = got
    ws, wL, wH, wst = want
    assert np.array_equal(L.view(np.uint32), np.asarray(wL).view(np.uint32)), (L, wL)
    assert np.array_equal(H.view(np.uint32), np.asarray(wH).view(np.uint32)), (H, wH)
    assert np.array_equal(s.view(np.uint32), np.asarray(ws).view(np.uint32))
    assert np.array_equal(st.view(np.uint64), np.asarray(wst, np.float64).view(np.uint64))


TRACK_CASES = [  # (outer, C, inner, G, with_perm, values)
    (2, 64, 256, 1, False, "t3"),          # one group, rows of 256
    (4, 96, 300, 3, True, "t3"),           # ragged rows, gather
    (3, 40, 7, 5, True, "normal"),         # inner not a multiple of 4 (element path)
    (8, 512, 1, 8, False, "t3"),           # channel axis contiguous
    (2, 128, 64, 20, True, "coarse"),      # more than 8 groups; many equal values (ties)
    (1, 33, 4, 32, False, "normal"),       # the largest group count, groups of 1-2 channels
]


def track_input(outer, C, inner, kind, seed):
    r = synth.rng(62, seed)
    if kind == "t3":
        x = r.standard_t(3, (outer, C, inner)) * np.exp(r.uniform(-3, 3, (1, C, 1)))
    elif kind == "coarse":
        x = np.round(r.standard_normal((outer, C, inner)) * 4) / 4   # few distinct values
    else:
        x = r.standard_normal((outer, C, inner))
    return x.astype(np.float32)


@pytest.mark.parametrize("outer,C,inner,G,with_perm,kind", TRACK_CASES)
def test_track_matches_oracle(dev, outer, C, inner, G, with_perm, kind):
    print(f"\n[track {outer}x{C}x{inner} G={G} perm={with_perm} {kind}]", flush=True)
    x = track_input(outer, C, inner, kind, C)
    r = synth.rng(63, C)
    group_of = r.integers(0, G, C).astype(np.uint8)
    group_of[:G] = np.arange(G)          # every group has a channel
    perm = r.permutation(C).astype(np.int32) if with_perm else None
    got = run_track(dev, x, group_of, G, perm=perm)
    s, L, H, st = oracle.softedge_track(x, group_of, G, perm=perm)
    check_track(got, (s, L, H, np.array(st)))


def test_track_ema_chain_empty_and_single_groups(dev):
    """Three batches continue one EMA state; group 3 has no channel (keeps its state), group 2 has
    a single value per batch; a group index past G counts as the last group."""
    print("\n[track ema chain]", flush=True)
    G, C = 5, 9
    group_of = np.array([0, 1, 0, 1, 4, 0, 1, 9, 2], np.uint8)   # 9 reads as group 4
    prev = np.array([[0.5, 9.0], [0.01, 2.0], [1.0, 1.0], [0.25, 4.0], [0.0, 0.0]], np.float64)
    state = [tuple(p) for p in prev]
    dstate = prev.copy()
    for k in range(3):
        x = track_input(1, C, 1 if k == 0 else 4, "t3", 100 + k)
        got = run_track(dev, x, group_of, G, prev=dstate)
        s, L, H, state = oracle.softedge_track(x, np.minimum(group_of, G - 1), G, prev=state)
        check_track(got, (s, L, H, np.array(state)))
        assert tuple(got[3][3]) == (0.25, 4.0)
        dstate = got[3]


def test_track_alpha_one_and_first_batch(dev):
    """alpha = 1 with a previous state gives the batch's own percentiles, as does no state."""
    x = track_input(2, 16, 64, "normal", 7)
    group_of = (np.arange(16) % 2).astype(np.uint8)
    a = run_track(dev, x, group_of, 2, prev=np.full((2, 2), 123.0), alpha=1.0)
    b = run_track(dev, x, group_of, 2)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ------------------------------------------------------------------------------------------------
# the Mamba1 scan with the variants

def layer(dev, inp, G, gs, **kw):
    import quantized_state_space_amd.workloads as wl
    return wl.Mamba1Layer(inp, G, gs, dev, with_h0=True, **kw)


def check_layer(lay, ref):
    import torch
    torch.cuda.synchronize()
    assert np.array_equal(lay.xs.cpu().numpy(), ref["xs"])
    assert np.array_equal(lay.sL.cpu().numpy(), ref["L"])
    assert np.array_equal(lay.sH.cpu().numpy(), ref["H"])
    assert np.array_equal(lay.xq.cpu().numpy(), ref["xq"])
    assert np.array_equal(lay.bs.cpu().numpy(), ref["bs"])
    assert np.array_equal(lay.cs.cpu().numpy(), ref["cs"])
    assert np.array_equal(lay.Bq.cpu().numpy().view(np.uint8), np.asarray(ref["Bq"]).view(np.uint8))
    assert np.array_equal(lay.Cq.cpu().numpy().view(np.uint8), np.asarray(ref["Cq"]).view(np.uint8))
    assert_rows_close(lay.y.cpu().numpy(), ref["y"], TOL_F32)
    assert_rows_close(lay.h_last.cpu().numpy(), ref["h_last"], TOL_F32, "h_last")


# gs = 4 with N = 16 stages fp16 code units (every wave's 4 states in one group); gs = 2 stages
# dequantized fp32 values
@pytest.mark.parametrize("x_ratio,bc_ratio,gs,N,L", [(2, 0, 4, 16, 300), (4, 4, 4, 16, 301),
                                                     (2, 2, 4, 16, 77), (4, 2, 2, 16, 130),
                                                     (2, 4, 8, 64, 129)])
def test_scan_soft_edge_variants(dev, x_ratio, bc_ratio, gs, N, L):
    import quantized_state_space_amd as qs
    print(f"\n[mamba1 x ratio {x_ratio}, B/C soft-edge {bc_ratio}, gs={gs} N={N} L={L}]", flush=True)
    form = {2: qs.QSSM_X_SOFTEDGE2, 4: qs.QSSM_X_SOFTEDGE}
    inp = synth.mamba1_inputs(cfg=12, batch=2, seqlen=L, dim=130, dstate=N, x_dist="student_t",
                              calib_batch=1, with_h0=True)
    lay = layer(dev, inp, G=4, gs=gs, x_code=form[x_ratio],
                bc_code=form[bc_ratio] if bc_ratio else qs.QSSM_X_INT8)
    lay.step()
    ref = op.mamba1(inp, G=4, gs=gs, soft_edge=True, with_h0=True, se_ratio=x_ratio,
                    bc_soft_edge=bc_ratio)
    check_layer(lay, ref)


def test_scan_tracked_thresholds_three_steps(dev):
    """The layer updates its x thresholds on the device before every encode; three steps on fresh
    x draws against the oracle's EMA chain from the same calibration state."""
    import torch
    import quantized_state_space_amd as qs
    print("\n[mamba1 tracked soft-edge thresholds]", flush=True)
    inp = synth.mamba1_inputs(cfg=13, batch=2, seqlen=256, dim=192, dstate=16, x_dist="student_t",
                              calib_batch=1, with_h0=True)
    lay = layer(dev, inp, G=4, gs=4, x_code=qs.QSSM_X_SOFTEDGE, track=True)
    calib = op.mamba1_calib(inp, G=4, gs=4, soft_edge=True)
    for k in range(3):
        step_inp = dict(inp)
        step_inp["x"] = synth.mamba1_inputs(cfg=20 + k, batch=2, seqlen=256, dim=192, dstate=16,
                                            x_dist="student_t", calib_batch=1)["x"]
        lay.x.copy_(torch.from_numpy(step_inp["x"]))
        lay.step()
        ref = op.mamba1(step_inp, G=4, gs=4, soft_edge=True, with_h0=True, calib=calib, track=True)
        check_layer(lay, ref)
        assert np.array_equal(lay.ema.cpu().numpy(), np.array(ref["se_state"]))
        calib = dict(calib, se_state=ref["se_state"])
