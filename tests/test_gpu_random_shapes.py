"""Seeded random shapes for every form against the oracle, to reach combinations the hand-picked
cases miss (sizes not multiples of the tiles, group counts, state sizes, output types)."""
import numpy as np
import pytest

import oracle
import oracle.pipelines as op
import qssm_synth as synth

pytestmark = pytest.mark.gpu

TOL = 2e-3


def rows_close(y, ref, tol, what):
    err = oracle.rowwise_error(y, ref)
    assert err.max() <= tol, f"{what}: max row error {err.max():.3e}"


@pytest.mark.parametrize("seed", range(8))
def test_mamba1_random(dev, seed):
    import torch
    import quantized_state_space_amd as qs
    import quantized_state_space_amd.workloads as wl
    r = np.random.default_rng(1000 + seed)
    N = int(r.choice([4, 8, 16, 32, 64]))
    gs = int(r.choice([g for g in (1, 2, 4, 8, 16) if N % g == 0]))
    B, D, L = int(r.integers(1, 4)), int(r.integers(1, 300)), int(r.integers(1, 400))
    G = int(r.integers(1, min(D, 16) + 1))
    soft = bool(r.integers(0, 2))
    yf16 = bool(r.integers(0, 2))
    print(f"\n[mamba1 random seed={seed}: B={B} D={D} L={L} N={N} gs={gs} G={G} soft={soft} "
          f"f16={yf16}]", flush=True)
    inp = synth.mamba1_inputs(cfg=300 + seed, batch=B, seqlen=L, dim=D, dstate=N, calib_batch=1,
                              with_h0=True, x_dist="student_t")
    lay = wl.Mamba1Layer(inp, G, gs, dev, x_code=qs.QSSM_X_SOFTEDGE if soft else qs.QSSM_X_INT8,
                         y_dtype=qs.QSSM_F16 if yf16 else qs.QSSM_F32, with_h0=True)
    lay.step()
    torch.cuda.synchronize()
    ref = op.mamba1(inp, G=G, gs=gs, soft_edge=soft, with_h0=True)
    assert np.array_equal(lay.xq.cpu().numpy().view(np.uint8), np.asarray(ref["xq"]).view(np.uint8))
    assert np.array_equal(lay.Bq.cpu().numpy(), ref["Bq"])
    rows_close(lay.y.float().cpu().numpy(), ref["y"], TOL, "y")
    rows_close(lay.h_last.cpu().numpy(), ref["h_last"], TOL, "h_last")


@pytest.mark.parametrize("seed", range(4))
def test_ssd_random(dev, seed):
    import torch
    import quantized_state_space_amd as qs
    import quantized_state_space_amd.workloads as wl
    r = np.random.default_rng(2000 + seed)
    Gbc = int(r.choice([1, 2, 4]))
    nh = Gbc * int(r.integers(1, 5))
    B, L = int(r.integers(1, 3)), int(r.integers(1, 700))
    gpb = int(r.choice([1, 2, 8]))
    yf16 = bool(r.integers(0, 2))
    h0 = bool(r.integers(0, 2))
    print(f"\n[ssd random seed={seed}: B={B} L={L} nh={nh} Gbc={Gbc} gpb={gpb} f16={yf16} "
          f"h0={h0}]", flush=True)
    inp = synth.ssd_inputs(cfg=400 + seed, batch=B, seqlen=L, nheads=nh, headdim=64, dstate=128,
                           ngroups=Gbc, calib_len=256, with_h0=h0)
    lay = wl.SsdLayer(inp, dev, y_dtype=qs.QSSM_F16 if yf16 else qs.QSSM_F32, with_h0=h0,
                      groups_per_block=gpb)
    lay.step()
    torch.cuda.synchronize()
    ref = op.ssd(inp, groups_per_block=gpb, with_h0=h0)
    assert np.array_equal(lay.xq.cpu().numpy(), ref["xq"])
    assert np.array_equal(lay.Bq.cpu().numpy(), ref["Bq"])
    assert np.array_equal(lay.Cq.cpu().numpy(), ref["Cq"])
    y = lay.y.float().cpu().numpy().astype(np.float64)
    rows_close(y.transpose(0, 2, 3, 1).reshape(-1, L),
               np.asarray(ref["y"], np.float64).transpose(0, 2, 3, 1).reshape(-1, L), TOL, "y")
    hl = lay.h_last.cpu().numpy()
    rows_close(hl.reshape(-1, 128), ref["h_last"].reshape(-1, 128), TOL, "h_last")


@pytest.mark.parametrize("seed", range(4))
def test_s4d_random(dev, seed):
    import torch
    import quantized_state_space_amd.workloads as wl
    r = np.random.default_rng(3000 + seed)
    shape = dict(batch=int(r.integers(1, 5)), seqlen=int(r.integers(1, 300)),
                 channels=int(r.integers(1, 9)), dstate=int(r.integers(1, 257)))
    print(f"\n[s4d random seed={seed}: {shape}]", flush=True)
    inp = synth.s4d_inputs(cfg=500 + seed, with_h0=True, **shape)
    lay = wl.S4dLayer(inp, dev, with_h0=True)
    lay.step()
    torch.cuda.synchronize()
    ref = op.s4d(inp, with_h0=True)
    rows_close(lay.y.cpu().numpy(), ref["y"], TOL, "y")
    hl = lay.h_last.cpu().numpy()
    rows_close(hl[..., 0] + 1j * hl[..., 1], ref["h_last"], TOL, "h_last")


@pytest.mark.parametrize("seed", range(4))
def test_decode_random(dev, seed):
    import torch
    import quantized_state_space_amd as qs
    import quantized_state_space_amd.workloads as wl
    r = np.random.default_rng(4000 + seed)
    N = int(r.choice([8, 16, 32, 64, 128, 256]))
    Gbc = int(r.choice([1, 2]))
    dims = dict(batch=int(r.integers(1, 6)), nheads=Gbc * int(r.integers(1, 4)),
                headdim=int(r.integers(1, 100)), dstate=N, ngroups=Gbc)
    f16 = bool(r.integers(0, 2))
    gs = min(N, 16)
    print(f"\n[decode random seed={seed}: {dims} f16={f16}]", flush=True)
    params = synth.decode_params(cfg=600 + seed, **dims)
    steps = [synth.decode_step_inputs(k, cfg=600 + seed, **dims) for k in range(3)]
    if f16:
        params["state0"] = params["state0"].astype(np.float16).astype(np.float32)
    lay = wl.DecodeLayer(params, dev, gs=gs, groups_per_block=1,
                         state_dtype=qs.QSSM_F16 if f16 else qs.QSSM_F32, emit_codes=True)
    ref = op.decode(params, steps, gs=gs, groups_per_block=1)
    tol = 1e-2 if f16 else TOL
    for k, s in enumerate(steps):
        lay.load_inputs(s)
        lay.step()
        torch.cuda.synchronize()
        for name, got in zip(("xq", "Bq", "Cq"), lay.codes):
            assert np.array_equal(got.cpu().numpy(), ref[name][k]), (name, k)
        rows_close(lay.y.cpu().numpy(), ref["y"][k], tol, "y")
    rows_close(lay.state.float().cpu().numpy(), ref["state"], tol, "state")
