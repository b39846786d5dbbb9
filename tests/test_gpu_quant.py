"""GPU parity of the quantizers and the soft-edge codec against the oracle: bit-exact codes,
through the C ABI."""
import numpy as np
import pytest

import oracle
import qssm_synth as synth

pytestmark = pytest.mark.gpu


def T(a, dev, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t if dtype is None else t.to(dtype)).to(dev)


def run_quant_x(dev, x, group_of, G, scales=None, perm=None, compute=False):
    import torch
    import quantized_state_space_amd as qs
    xt = T(x, dev)
    q = torch.empty(x.shape, dtype=torch.int8, device=dev)
    s = T(np.ones(G, np.float32) if scales is None else scales, dev)
    qs.qssm_quant_group_x(xt, T(group_of, dev), G, s, q, perm=None if perm is None else T(perm, dev),
                          compute_scales=compute)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


CASES = [  # (outer, C, inner, G, with_perm)
    (1, 64, 256, 1, False),     # tiny Mamba1 x
    (2, 100, 300, 3, True),     # ragged rows, gather
    (3, 37, 5, 4, True),        # inner not a multiple of 16
    (16, 8192, 1, 64, False),   # SSD-shaped x (channel axis contiguous)
    (5, 129, 1, 7, True),       # channel axis contiguous with a gather
    (1, 1, 17, 1, False),
    (2, 600, 12, 256, True),    # the largest group count
]


@pytest.mark.parametrize("outer,C,inner,G,with_perm", CASES)
def test_quant_group_x_bit_exact(dev, outer, C, inner, G, with_perm):
    print(f"\n[quant_group_x] outer={outer} C={C} inner={inner} G={G} perm={with_perm}", flush=True)
    r = np.random.default_rng(outer * 1000 + C)
    x = (r.standard_t(3, (outer, C, inner)) * np.where(r.random((outer, C, inner)) < 0.01, 50, 1)).astype(np.float32)
    x.flat[::97] = np.nan
    x.flat[5::211] = np.inf
    x.flat[7::307] = -np.inf
    group_of = r.integers(0, G, C).astype(np.uint8)
    perm = r.permutation(C).astype(np.int32) if with_perm else None
    # static scales
    scales = r.uniform(0.01, 0.2, G).astype(np.float32)
    q, _ = run_quant_x(dev, x, group_of, G, scales, perm)
    assert np.array_equal(q, oracle.quant_group_x(x, group_of, scales, perm=perm))
    # scales computed on the device from the tensor itself
    q2, s2 = run_quant_x(dev, x, group_of, G, None, perm, compute=True)
    want_s = oracle.group_scales(x, group_of, G, perm)
    assert np.array_equal(s2, want_s)
    assert np.array_equal(q2, oracle.quant_group_x(x, group_of, want_s, perm=perm))


def test_quant_adversarial_ties_and_specials(dev):
    print("\n[quant adversarial]", flush=True)
    for s in (np.float32(0.0371), np.float32(1.0), np.float32(3.0) / np.float32(7.0),
              np.float32(2.0 ** -99), np.float32(2.0 ** 99)):
        v = synth.quantizer_edge_values(scale=s, n=4096)
        x = v.reshape(1, 1, -1)
        q, _ = run_quant_x(dev, x, np.zeros(1, np.uint8), 1, np.array([s], np.float32))
        assert np.array_equal(q.ravel(), oracle.quant_code(v, s)), float(s)
    for bad in (0.0, -1.0, np.nan, np.inf, 2.0 ** -101, 2.0 ** 101):
        q, _ = run_quant_x(dev, np.ones((1, 1, 32), np.float32), np.zeros(1, np.uint8), 1,
                           np.array([bad], np.float32))
        assert not q.any()


def test_quant_empty_tensor(dev):
    import torch
    import quantized_state_space_amd as qs
    x = torch.empty((0, 8, 4), dtype=torch.float32, device=dev)
    q = torch.empty((0, 8, 4), dtype=torch.int8, device=dev)
    s = torch.zeros(2, dtype=torch.float32, device=dev)
    qs.qssm_quant_group_x(x, T(np.zeros(8, np.uint8), dev), 2, s, q, compute_scales=True)
    torch.cuda.synchronize()
    assert s.cpu().tolist() == [1.0, 1.0]


# (the last two have more scales than the LDS table holds: the scales are read from memory)
@pytest.mark.parametrize("outer,Gbc,N,inner,gs", [(1, 1, 16, 256, 4), (2, 8, 128, 1, 16),
                                                  (3, 2, 12, 33, 3), (64, 8, 128, 1, 128),
                                                  (2, 16, 128, 8, 1), (3, 9, 256, 1, 2)])
def test_quant_state_group_bit_exact(dev, outer, Gbc, N, inner, gs):
    import torch
    import quantized_state_space_amd as qs
    print(f"\n[quant_state_group] {outer}x{Gbc}x{N}x{inner} gs={gs}", flush=True)
    r = np.random.default_rng(N * 7 + inner)
    bc = r.standard_normal((outer, Gbc, N, inner)).astype(np.float32)
    bc.flat[3::101] = np.nan
    scales = r.uniform(0.005, 0.05, Gbc * N // gs).astype(np.float32)
    q = torch.empty(bc.shape, dtype=torch.int8, device=dev)
    st = T(scales, dev)
    qs.qssm_quant_state_group_BC(T(bc, dev), gs, st, q)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), oracle.quant_state_group(bc, gs, scales))
    st2 = torch.zeros(Gbc * N // gs, dtype=torch.float32, device=dev)
    qs.qssm_quant_state_group_BC(T(bc, dev), gs, st2, q, compute_scales=True)
    torch.cuda.synchronize()
    want = oracle.state_group_scales(bc, gs)
    assert np.array_equal(st2.cpu().numpy(), want)
    assert np.array_equal(q.cpu().numpy(), oracle.quant_state_group(bc, gs, want))


def test_softedge_encode_decode_bit_exact(dev):
    import torch
    import quantized_state_space_amd as qs
    print("\n[softedge]", flush=True)
    r = np.random.default_rng(31)
    outer, C, inner, G = 2, 96, 200, 3
    x = (r.standard_t(3, (outer, C, inner))).astype(np.float32)
    x.flat[::89] = np.nan
    x.flat[1::173] = np.inf
    x.flat[2::179] = -np.inf
    x.flat[3::181] = -0.0
    group_of = r.integers(0, G, C).astype(np.uint8)
    perm = r.permutation(C).astype(np.int32)
    s = np.array([0.05, 0.02, 0.3], np.float32)
    L = np.array([0.1, 0.0, 0.5], np.float32)
    H = np.array([3.0, 1.0, 0.2], np.float32)   # group 2 has L > H (standard case)
    code = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    qs.qssm_softedge_encode(T(x, dev), T(group_of, dev), G, T(s, dev), T(L, dev), T(H, dev), code,
                            perm=T(perm, dev))
    out = torch.empty(x.shape, dtype=torch.float32, device=dev)
    qs.qssm_softedge_decode(code, T(group_of, dev), G, T(s, dev), out)
    torch.cuda.synchronize()
    want = oracle.softedge_encode(x, group_of, s, L, H, perm=perm)
    got = code.cpu().numpy()
    assert np.array_equal(got, want)
    dec = oracle.softedge_decode_f32(want, group_of, s)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), dec.view(np.uint32))


def test_softedge_decode_all_bytes(dev):
    import torch
    import quantized_state_space_amd as qs
    scales = np.array([1.0, 0.0173, 2.0 ** -90, 3.3e20, 0.0], np.float32)
    codes = np.tile(np.arange(256, dtype=np.uint8), (1, len(scales), 1))
    out = torch.empty(codes.shape, dtype=torch.float32, device=dev)
    qs.qssm_softedge_decode(T(codes, dev), T(np.arange(len(scales), dtype=np.uint8), dev),
                            len(scales), T(scales, dev), out)
    torch.cuda.synchronize()
    want = np.stack([oracle.softedge_value_table(s).astype(np.float32) for s in scales])[None]
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
