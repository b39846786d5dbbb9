"""GPU parity of the Mamba2 SSD chunked int8 path against the oracle: codes bit-exact, outputs and
final state within the fp32-state tolerance per (b, head, channel) row over time. The default chunk
state (fp16 operands, fp32 accumulate) is compared with the oracle's exact chunked form; the
requantized int8 chunk state is pinned in its exact special case (A = 0 and constant delta, where
the requantization ratio is exactly one) and otherwise held to its accuracy against the exact form."""
import numpy as np
import pytest

import oracle
import oracle.pipelines as op
import qssm_synth as synth

pytestmark = pytest.mark.gpu

TOL = 2e-3


def run_layer(dev, inp, **kw):
    import torch
    import quantized_state_space_amd.workloads as wl
    lay = wl.SsdLayer(inp, dev, **kw)
    lay.step()
    torch.cuda.synchronize()
    return lay


def y_rows(y):
    """[B, L, nh, P] -> rows (b, h, p) over t."""
    y = np.asarray(y, dtype=np.float64)
    return y.transpose(0, 2, 3, 1).reshape(-1, y.shape[1])


def check(lay, ref, heads=None, tol=TOL, tol_h=TOL):
    assert np.array_equal(lay.group_of, ref["group_of"])
    assert np.array_equal(lay.xs.cpu().numpy(), ref["xs"])
    assert np.array_equal(lay.bs.cpu().numpy(), ref["bs"])
    assert np.array_equal(lay.cs.cpu().numpy(), ref["cs"])
    assert np.array_equal(lay.xq.cpu().numpy(), ref["xq"])
    assert np.array_equal(lay.Bq.cpu().numpy(), ref["Bq"])
    assert np.array_equal(lay.Cq.cpu().numpy(), ref["Cq"])
    y = lay.y.float().cpu().numpy()
    hl = lay.h_last.cpu().numpy()
    if heads is not None:
        y, hl = y[:, :, heads], hl[:, heads]
    ey = oracle.rowwise_error(y_rows(y), y_rows(ref["y"]))
    eh = oracle.rowwise_error(hl.reshape(-1, hl.shape[-1]), ref["h_last"].reshape(-1, hl.shape[-1]))
    print(f"  max row error y {ey.max():.2e}, h_last {eh.max():.2e}", flush=True)
    assert ey.max() <= tol, ey.max()
    if tol_h is not None:
        assert eh.max() <= tol_h, eh.max()
    return y


@pytest.mark.parametrize("L,with_h0", [(600, True), (256, False), (100, True), (1, False)])
def test_ssd_small(dev, L, with_h0):
    print(f"\n[ssd small L={L} h0={with_h0}]", flush=True)
    inp = synth.ssd_inputs(cfg=41, batch=2, seqlen=L, nheads=4, headdim=64, dstate=128, ngroups=2,
                           calib_len=256, with_h0=with_h0)
    lay = run_layer(dev, inp, with_h0=with_h0)
    ref = op.ssd(inp, with_h0=with_h0)
    y = check(lay, ref)
    seq = op.ssd(inp, with_h0=with_h0, exact=True)
    e = oracle.rowwise_error(y_rows(y), y_rows(seq["y"])).max()
    print(f"  vs the sequential scan: max row error {e:.2e}", flush=True)


def test_ssd_odd_heads_per_group(dev):
    """Three heads per B/C group in two groups: the second half of each group's last pair of heads
    has no head of its own and repeats the first's work; an odd, ragged number of chunks (520
    steps: 3 chunks, the last of 8 steps), whose next-chunk loads run past the sequence."""
    print("\n[ssd 3 heads per group, L=520]", flush=True)
    inp = synth.ssd_inputs(cfg=49, batch=3, seqlen=520, nheads=6, headdim=64, dstate=128,
                           ngroups=2, calib_len=256, with_h0=True)
    lay = run_layer(dev, inp, with_h0=True)
    ref = op.ssd(inp, with_h0=True)
    check(lay, ref)


def special_case_inputs(cfg, L, with_h0, kind):
    """A = 0, so every decay factor is exactly one and w_j = delta_j. kind "const": a per-head
    constant delta, the requantization ratio w_j / w_max is exactly one and the requantized operand
    is the x code. kind "pow2": delta drawn from {2^-4, ..., 2^-7}, every ratio is an exact power of
    two, so qx * ratio is exact in any precision and both sides take the same rounding decisions,
    ties to even included."""
    inp = synth.ssd_inputs(cfg=cfg, batch=2, seqlen=L, nheads=4, headdim=64, dstate=128, ngroups=2,
                           calib_len=256, with_h0=with_h0)
    inp["A"] = np.zeros_like(inp["A"])
    if kind == "const":
        inp["delta"] = np.broadcast_to(np.float32([0.01, 0.02, 0.05, 0.1]),
                                       inp["delta"].shape).astype(np.float32).copy()
    else:
        e = synth.rng(cfg, 99).integers(4, 8, size=inp["delta"].shape)
        inp["delta"] = np.ldexp(np.float32(1.0), -e).astype(np.float32)
    return inp


@pytest.mark.parametrize("L,with_h0,kind", [(600, True, "const"), (256, False, "pow2"),
                                            (700, True, "pow2")])
def test_ssd_int8_state_special_case(dev, L, with_h0, kind):
    import quantized_state_space_amd as qs
    print(f"\n[ssd int8 chunk state, A=0, {kind} delta, L={L}]", flush=True)
    inp = special_case_inputs(44, L, with_h0, kind)
    lay = run_layer(dev, inp, with_h0=with_h0, state_mma=qs.QSSM_MMA_I8)
    ref = op.ssd(inp, with_h0=with_h0, int8_state=True)
    check(lay, ref)


@pytest.mark.parametrize("cfg,L", [(45, 600), (48, 1000)])
def test_ssd_int8_state_generic(dev, cfg, L):
    """Generic inputs: the requantized chunk state rounds qx * w_j / w_max to int8. The kernel takes
    the weights, their maximum and the rounding decisions in fp64, as the oracle does (only the
    order of the cumulative sum differs, by a few fp64 units), so both sides pick the same codes
    and y and h_last are held to the fp32-state tolerance against the oracle's int8 mode."""
    import quantized_state_space_amd as qs
    print(f"\n[ssd int8 chunk state generic cfg={cfg} L={L}]", flush=True)
    inp = synth.ssd_inputs(cfg=cfg, batch=2, seqlen=L, nheads=4, headdim=64, dstate=128,
                           ngroups=2, calib_len=256, with_h0=True)
    lay = run_layer(dev, inp, with_h0=True, state_mma=qs.QSSM_MMA_I8)
    ref = op.ssd(inp, with_h0=True, int8_state=True)
    check(lay, ref)


def test_ssd_invalid_scales_one_head_per_group(dev):
    """One head per B/C group (the head loops run once), and scales outside [2^-100, 2^100]: an x
    group (its channels then carry only the inter-chunk state and no D term), a B state group and a
    C state group contribute zeros. The group map and scales are the oracle's own calibration with
    three scales replaced; both sides take them."""
    import torch
    print("\n[ssd invalid scales, one head per group]", flush=True)
    inp = synth.ssd_inputs(cfg=47, batch=2, seqlen=300, nheads=3, headdim=64, dstate=128,
                           ngroups=3, calib_len=256, with_h0=True)
    cal = op.ssd(inp, with_h0=True, heads=np.array([0]))
    group_of = cal["group_of"].copy()
    xs, bs, cs = (cal[k].copy() for k in ("xs", "bs", "cs"))
    xs[2] = 0.0
    bs[5] = np.float32(1e-35)
    cs[9] = np.float32(2.0 ** 101)
    import quantized_state_space_amd.workloads as wl
    lay = wl.SsdLayer(inp, dev, with_h0=True)
    lay.group_of = group_of
    for t, v in ((lay.group_t, group_of), (lay.xs, xs), (lay.bs, bs), (lay.cs, cs)):
        t.copy_(torch.from_numpy(v))
    lay.step()
    torch.cuda.synchronize()
    ref = op.ssd(inp, with_h0=True, calib=(group_of, xs, bs, cs))
    check(lay, ref)


def test_ssd_bad_state_mma(dev):
    import quantized_state_space_amd as qs
    inp = synth.ssd_inputs(cfg=46, batch=1, seqlen=64, nheads=4, headdim=64, dstate=128, ngroups=2,
                           calib_len=256)
    import quantized_state_space_amd.workloads as wl
    with pytest.raises(qs.QssmError, match="state_mma"):
        wl.SsdLayer(inp, dev, state_mma=7).step()


def test_ssd_fp16_output(dev):
    import quantized_state_space_amd as qs
    print("\n[ssd fp16 y]", flush=True)
    inp = synth.ssd_inputs(cfg=42, batch=1, seqlen=512, nheads=8, headdim=64, dstate=128,
                           ngroups=1, calib_len=256)
    lay = run_layer(dev, inp, y_dtype=qs.QSSM_F16)
    ref = op.ssd(inp)
    check(lay, ref)


def test_ssd_determinism(dev):
    import torch
    print("\n[ssd determinism]", flush=True)
    inp = synth.ssd_inputs(cfg=43, batch=1, seqlen=700, nheads=16, headdim=64, dstate=128,
                           ngroups=2, calib_len=256, with_h0=True)
    lay = run_layer(dev, inp, with_h0=True)
    y1, h1 = lay.y.clone(), lay.h_last.clone()
    lay.scan()
    torch.cuda.synchronize()
    assert torch.equal(lay.y, y1) and torch.equal(lay.h_last, h1)


def test_ssd_full_size_sampled_heads(dev):
    """Mamba2-8B-shaped layer (B=4, L=4096, 128 heads x 64, N=128, 8 groups, chunk 256), launched as
    the benchmark does: all codes bit-exact, y and h_last of sampled heads against the oracle."""
    print("\n[ssd full size]", flush=True)
    inp = synth.ssd_inputs(cfg=4, calib_len=256)
    lay = run_layer(dev, inp)
    heads = np.array([0, 37, 127])
    ref = op.ssd(inp, heads=heads)
    check(lay, ref, heads=heads)


def test_ssd_empty_sequence(dev):
    """L = 0: no chunk, nothing read or written per step, h_last = h0 exactly."""
    import torch
    import quantized_state_space_amd as qs
    print("\n[ssd L=0]", flush=True)
    B, nh, P, N, Gbc = 2, 16, 64, 128, 2
    g = torch.Generator().manual_seed(6)
    h0 = torch.randn((B, nh, P, N), generator=g).to(dev)
    h_last = torch.full_like(h0, float("nan"))
    xq = torch.empty((B, 0, nh, P), dtype=torch.int8, device=dev)
    bc = torch.empty((B, 0, Gbc, N), dtype=torch.int8, device=dev)
    sc = torch.ones(Gbc * N // 16, device=dev)
    a = qs.ssd_args(xq, torch.zeros(nh * P, dtype=torch.uint8, device=dev), torch.ones(1, device=dev),
                    torch.empty((B, 0, nh), device=dev), -torch.ones(nh, device=dev), bc, bc, sc, sc,
                    16, 256, torch.empty((B, 0, nh, P), device=dev), h0=h0, h_last=h_last)
    ws = torch.empty(max(qs.qssm_ssd_workspace_size(a), 1), dtype=torch.uint8, device=dev)
    qs.qssm_ssd_chunk_int8(a, ws)
    torch.cuda.synchronize()
    assert torch.equal(h_last, h0)
