"""GPU parity of the Mamba1 W8A8 selective scan (quantize x, B, C, then scan) against the oracle:
bit-exact codes and scales, outputs within the fp32-state tolerance per (b, channel) row."""
import numpy as np
import pytest

import oracle
import oracle.pipelines as op
import qssm_synth as synth

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-3   # max relative error per row, fp32 state
TOL_F16_OUT = 2e-3  # fp16 output rounding (2^-11 relative) stays inside the same bar


def layer(dev, inp, G, gs, **kw):
    import quantized_state_space_amd.workloads as wl
    return wl.Mamba1Layer(inp, G, gs, dev, **kw)


def check_codes(lay, ref, soft_edge=False):
    import torch
    torch.cuda.synchronize()
    assert np.array_equal(lay.perm, ref["perm"]) and np.array_equal(lay.group_of, ref["group_of"])
    assert np.array_equal(lay.xs.cpu().numpy(), ref["xs"])
    assert np.array_equal(lay.bs.cpu().numpy(), ref["bs"])
    assert np.array_equal(lay.cs.cpu().numpy(), ref["cs"])
    got_x = lay.xq.cpu().numpy()
    assert np.array_equal(got_x.view(np.uint8), np.asarray(ref["xq"]).view(np.uint8))
    assert np.array_equal(lay.Bq.cpu().numpy(), ref["Bq"])
    assert np.array_equal(lay.Cq.cpu().numpy(), ref["Cq"])


def assert_rows_close(y, ref, tol, what="y"):
    err = oracle.rowwise_error(y, ref)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol, f"{what}: max row error {err.max():.3e} at row {worst}"
    return err.max()


def test_c1_tiny_dynamic_scales(dev):
    """Tiny Mamba1 layer: B=1, L=256, D=64, N=16, per-tensor x scale, 4 state groups of 4, scales
    from the tensors themselves (computed on the device)."""
    print("\n[c1 tiny mamba1]", flush=True)
    inp = synth.c1_inputs()
    lay = layer(dev, inp, G=1, gs=4, dynamic_scales=True)
    lay.step()
    ref = op.mamba1(inp, G=1, gs=4, dynamic=True)
    check_codes(lay, ref)
    assert_rows_close(lay.y.cpu().numpy(), ref["y"], TOL_F32)
    assert_rows_close(lay.h_last.cpu().numpy(), ref["h_last"], TOL_F32, "h_last")


# gs: B/C state-group size. The kernel stages B/C as fp16 codes when each wave's states lie in one
# group (gs a multiple of the states per wave: 4, or 2 for N = 8, or 8 for N = 64) and as
# dequantized fp32 values otherwise; both layouts are covered.
@pytest.mark.parametrize("B,D,L,N,G,soft,gs", [(2, 100, 300, 16, 3, False, 4),
                                                (1, 64, 77, 4, 2, False, 4),
                                                (2, 192, 64, 8, 5, False, 4),
                                                (1, 128, 200, 32, 4, False, 4),
                                                (1, 64, 129, 64, 2, False, 4),
                                                (1, 64, 129, 64, 2, False, 16),
                                                (2, 100, 300, 16, 3, False, 2),
                                                (1, 64, 70, 16, 2, False, 16),
                                                (2, 130, 301, 16, 4, True, 4),
                                                (1, 70, 99, 16, 3, True, 1)])
@pytest.mark.parametrize("tb", [0, 1])  # the library's choice (time windows here), the chain form
def test_ragged_shapes_static_scales(dev, B, D, L, N, G, soft, gs, tb):
    print(f"\n[mamba1 B={B} D={D} L={L} N={N} G={G} softedge={soft} gs={gs} tb={tb}]", flush=True)
    import quantized_state_space_amd as qs
    inp = synth.mamba1_inputs(cfg=11, batch=B, seqlen=L, dim=D, dstate=N, x_dist="student_t",
                              calib_batch=1, with_h0=True)
    xc = qs.QSSM_X_SOFTEDGE if soft else qs.QSSM_X_INT8
    lay = layer(dev, inp, G=G, gs=gs, x_code=xc, with_h0=True, time_blocks=tb)
    lay.step()
    ref = op.mamba1(inp, G=G, gs=gs, soft_edge=soft, with_h0=True)
    if soft:
        assert np.array_equal(lay.sL.cpu().numpy(), ref["L"])
        assert np.array_equal(lay.sH.cpu().numpy(), ref["H"])
    check_codes(lay, ref)
    assert_rows_close(lay.y.cpu().numpy(), ref["y"], TOL_F32)
    assert_rows_close(lay.h_last.cpu().numpy(), ref["h_last"], TOL_F32, "h_last")


@pytest.mark.parametrize("code16", [True, False])
def test_invalid_scales_zero_their_values(dev, code16):
    """A group whose scale is outside [2^-100, 2^100] contributes zeros: an x group (its channels
    then only carry the decaying initial state), a B state group and a C state group."""
    import torch
    print(f"\n[mamba1 invalid scales code16={code16}]", flush=True)
    gs = 4 if code16 else 2
    inp = synth.mamba1_inputs(cfg=14, batch=2, seqlen=150, dim=128, dstate=16, calib_batch=1,
                              with_h0=True)
    lay = layer(dev, inp, G=4, gs=gs, with_h0=True)
    cal = op.mamba1_calib(inp, 4, gs)
    assert np.array_equal(lay.xs.cpu().numpy(), cal["xs"])
    cal["xs"] = cal["xs"].copy(); cal["xs"][1] = 0.0
    cal["bs"] = cal["bs"].copy(); cal["bs"][2] = np.float32(1e-35)
    cal["cs"] = cal["cs"].copy(); cal["cs"][0] = np.float32(2.0 ** 101)
    for t, v in ((lay.xs, cal["xs"]), (lay.bs, cal["bs"]), (lay.cs, cal["cs"])):
        t.copy_(torch.from_numpy(v))
    lay.step()
    ref = op.mamba1(inp, G=4, gs=gs, with_h0=True, calib=cal)
    check_codes(lay, ref)
    assert_rows_close(lay.y.cpu().numpy(), ref["y"], TOL_F32)
    assert_rows_close(lay.h_last.cpu().numpy(), ref["h_last"], TOL_F32, "h_last")


def test_fp16_output(dev):
    import quantized_state_space_amd as qs
    print("\n[mamba1 fp16 y]", flush=True)
    inp = synth.mamba1_inputs(cfg=12, batch=1, seqlen=160, dim=64, dstate=16, calib_batch=1)
    lay = layer(dev, inp, G=2, gs=4, y_dtype=qs.QSSM_F16)
    lay.step()
    ref = op.mamba1(inp, G=2, gs=4)
    assert_rows_close(lay.y.float().cpu().numpy(), ref["y"], TOL_F16_OUT)


def test_split_resume_and_determinism(dev):
    """scan(L) == scan(L1) then scan(L2, h0 = h_last); two runs are bitwise identical."""
    import torch
    import quantized_state_space_amd as qs
    print("\n[mamba1 resume]", flush=True)
    inp = synth.mamba1_inputs(cfg=13, batch=2, seqlen=96, dim=64, dstate=16, calib_batch=1)
    lay = layer(dev, inp, G=2, gs=4)
    lay.step()
    torch.cuda.synchronize()
    y_full, h_full = lay.y.clone(), lay.h_last.clone()
    lay.scan()
    torch.cuda.synchronize()
    assert torch.equal(lay.y, y_full) and torch.equal(lay.h_last, h_full)
    L1 = 40
    outs = []
    h0 = None
    for sl in (slice(0, L1), slice(L1, 96)):
        xq = lay.xq[..., sl].contiguous()
        y = torch.empty_like(xq, dtype=torch.float32)
        hl = torch.empty_like(h_full)
        a = qs.scan_args(xq, qs.QSSM_X_INT8, lay.group_t, lay.xs, lay.delta[..., sl].contiguous(),
                         lay.A, lay.Bq[..., sl].contiguous(), lay.Cq[..., sl].contiguous(), lay.bs,
                         lay.cs, 4, y, Dskip=lay.D, h0=h0, h_last=hl)
        ws = torch.empty(qs.qssm_scan_workspace_size(a), dtype=torch.uint8, device=dev)
        qs.qssm_scan_w8a8(a, ws)
        outs.append(y)
        h0 = hl
    torch.cuda.synchronize()
    y2 = torch.cat(outs, dim=-1).cpu().numpy()
    assert_rows_close(y2, y_full.cpu().numpy().astype(np.float64), 1e-5)
    assert_rows_close(h0.cpu().numpy(), h_full.cpu().numpy().astype(np.float64), 1e-5)


@pytest.mark.parametrize("soft", [False, True])
def test_c3_full_size_sampled(dev, soft):
    """Mamba1-130M-shaped layer (B=8, L=2048, D=1536, N=16, 8 clustered x groups), launched exactly
    as the benchmark does: every code bit-exact, y and h_last checked on sampled (b, channel) rows."""
    import quantized_state_space_amd as qs
    print(f"\n[c3 full size softedge={soft}]", flush=True)
    inp = synth.c3_inputs()
    lay = layer(dev, inp, G=8, gs=4, x_code=qs.QSSM_X_SOFTEDGE if soft else qs.QSSM_X_INT8)
    lay.step()
    r = np.random.default_rng(3)
    bsel = np.repeat(np.arange(8), 6)
    dsel = np.concatenate([r.choice(1536, 6, replace=False) for _ in range(8)])
    dsel[:2] = [0, 1535]
    ref = op.mamba1(inp, G=8, gs=4, soft_edge=soft, rows=(bsel, dsel))
    check_codes(lay, ref)
    y = lay.y.cpu().numpy()[bsel, dsel]
    h = lay.h_last.cpu().numpy()[bsel, dsel]
    assert_rows_close(y, ref["y_rows"], TOL_F32)
    assert_rows_close(h, ref["h_rows"], TOL_F32, "h_last")


def test_empty_sequence(dev):
    """L = 0: nothing is read or written per step (those buffers are empty), h_last = h0."""
    import torch
    import quantized_state_space_amd as qs
    print("\n[mamba1 L=0]", flush=True)
    B, D, N = 2, 96, 16
    g = torch.Generator().manual_seed(5)
    A = (-torch.rand((D, N), generator=g) - 0.1).to(dev)
    h0 = torch.randn((B, D, N), generator=g).to(dev)
    h_last = torch.full((B, D, N), float("nan"), device=dev)
    e8 = torch.empty((B, D, 0), dtype=torch.int8, device=dev)
    ebc = torch.empty((B, 1, N, 0), dtype=torch.int8, device=dev)
    one = torch.ones(N // 4, device=dev)
    a = qs.scan_args(e8, qs.QSSM_X_INT8, torch.zeros(D, dtype=torch.uint8, device=dev),
                     torch.ones(1, device=dev), torch.empty((B, D, 0), device=dev), A, ebc, ebc,
                     one, one, 4, torch.empty((B, D, 0), device=dev), h0=h0, h_last=h_last)
    ws = torch.empty(qs.qssm_scan_workspace_size(a), dtype=torch.uint8, device=dev)
    qs.qssm_scan_w8a8(a, ws)
    torch.cuda.synchronize()
    torch.testing.assert_close(h_last, h0, rtol=1e-6, atol=0)


@pytest.mark.parametrize("D,N,Gbc", [(256, 16, 4), (128, 8, 2), (192, 32, 3)])
def test_several_bc_groups(dev, D, N, Gbc):
    """B and C with several groups, each shared by D / Gbc consecutive channels (multiples of 64:
    one workgroup's channels share one group). Scales from the tensors themselves, channels in
    their original order (a cluster permutation would have to stay inside each B/C group)."""
    print(f"\n[mamba1 D={D} N={N} Gbc={Gbc}]", flush=True)
    inp = synth.mamba1_inputs(cfg=24, batch=2, seqlen=200, dim=D, dstate=N, bc_groups=Gbc)
    lay = layer(dev, inp, G=2, gs=4 if N >= 4 else N, dynamic_scales=True, perm=False)
    lay.step()
    ref = op.mamba1(inp, G=2, gs=4 if N >= 4 else N, dynamic=True)
    check_codes(lay, ref)
    assert_rows_close(lay.y.cpu().numpy(), ref["y"], TOL_F32)
    assert_rows_close(lay.h_last.cpu().numpy(), ref["h_last"], TOL_F32, "h_last")


@pytest.mark.parametrize("sxb,sc", [(2.0 ** -80, 2.0 ** 70), (2.0 ** 70, 2.0 ** -70)])
def test_scan_extreme_valid_scales(dev, sxb, sc):
    """x and B scales that are valid on their own but whose product leaves the normal fp32 range
    (2^-160, 2^140), with a C scale that brings y back into range. The fp16-code chains run in
    units of that product, so the kernel keeps it as a significand and an exponent. No D term, so
    y is the state readout alone; h_last itself is outside the fp32 range here and not compared."""
    import torch
    print(f"\n[scan extreme scales sx = sB = {sxb:g}, sC = {sc:g}]", flush=True)
    inp = synth.mamba1_inputs(cfg=71, batch=2, seqlen=100, dim=64, dstate=16, calib_batch=1)
    inp["D"] = np.zeros_like(inp["D"])
    cal = op.mamba1_calib(inp, 2, 4)
    cal["xs"] = np.full_like(cal["xs"], sxb)
    cal["bs"] = np.full_like(cal["bs"], sxb)
    cal["cs"] = np.full_like(cal["cs"], sc)
    lay = layer(dev, inp, G=2, gs=4)
    for t, v in ((lay.xs, cal["xs"]), (lay.bs, cal["bs"]), (lay.cs, cal["cs"])):
        t.copy_(torch.from_numpy(v))
    lay.step()
    ref = op.mamba1(inp, G=2, gs=4, calib=cal)
    check_codes(lay, ref)
    y = lay.y.cpu().numpy()
    assert np.all(np.isfinite(y))
    e = assert_rows_close(y, ref["y"], TOL_F32)
    print(f"  max row error y {e:.2e}", flush=True)
