"""GPU parity of the W4A8 linear layer (Quamba2 abstract: W4A8 for large-batch decoding) against
the oracle: activation codes bit-exact (the library quantizer), weight scales and codes bit-exact
(the host quantizer, checked on the CPU in test_capi), and y per row within the error of the fp32
scaling of exact int32 group sums: at most (groups + 2) fp32 roundings of the largest term, held to
1e-5 of the row (fp32 y) or the fp16 rounding (2^-11) for fp16 y."""
import numpy as np
import pytest

import oracle
import qssm_synth as synth

pytestmark = pytest.mark.gpu


def run(dev, M, N, K, group, seed, bias=True, f16=False):
    import torch
    import quantized_state_space_amd as qs
    import quantized_state_space_amd.workloads as wl
    inp = synth.w4a8_inputs(cfg=seed, M=M, N=N, K=K)
    lay = wl.W4A8Linear(inp["w"], inp["x"], inp["x_cal"], dev, group=group,
                        bias=inp["bias"] if bias else None,
                        y_dtype=qs.QSSM_F16 if f16 else qs.QSSM_F32)
    lay.step()
    torch.cuda.synchronize()
    return inp, lay


def oracle_ref(inp, group, bias=True, rows=None):
    x = inp["x"] if rows is None else inp["x"][rows]
    sa = oracle.scale_from_absmax(oracle.finite_absmax(inp["x_cal"].reshape(1, -1), axis=1))[0]
    qa = oracle.quant_group_x(x.reshape(1, 1, -1), np.zeros(1, np.uint8), [sa]).reshape(x.shape)
    sw = oracle.w4_scales(inp["w"], group)
    qw = oracle.quant_w4(inp["w"], group, sw)
    y = oracle.gemm_w4a8(qa, sa, qw, sw, group, inp["bias"].astype(np.float64) if bias else None)
    return qa, sa, sw, y


@pytest.mark.parametrize("M,N,K,group,bias,f16", [(77, 130, 192, 64, True, False),
                                                  (128, 128, 256, 256, False, False),
                                                  (1, 300, 512, 128, True, False),
                                                  (300, 65, 128, 128, True, True),
                                                  (256, 512, 1024, 64, True, False),
                                                  # the wide-tile form (M >= 1024, one scale per
                                                  # output channel): ragged row and column tiles
                                                  (1100, 300, 256, 256, True, False),
                                                  (1030, 520, 512, 512, False, True),
                                                  # the few-token form (loads four K steps of 128
                                                  # ahead): 128-row tiles, 64-row tiles (M <= 64),
                                                  # one and two rounds of four steps, 64-column
                                                  # tiles (more than 256 tiles of 128 columns)
                                                  (77, 130, 512, 512, True, True),
                                                  (200, 260, 1024, 1024, True, False),
                                                  (33, 300, 512, 512, False, False),
                                                  (64, 257, 1024, 1024, True, True),
                                                  (130, 16450, 512, 512, True, False)])
def test_w4a8_small(dev, M, N, K, group, bias, f16):
    print(f"\n[w4a8 M={M} N={N} K={K} group={group} bias={bias} f16={f16}]", flush=True)
    inp, lay = run(dev, M, N, K, group, 61, bias, f16)
    qa, sa, sw, y = oracle_ref(inp, group, bias)
    assert np.array_equal(lay.xq.cpu().numpy(), qa)
    assert lay.xs.cpu().numpy()[0] == sa
    assert np.array_equal(lay.w_scales_host, sw)
    got = lay.y.float().cpu().numpy()
    e = oracle.rowwise_error(got, y).max()
    print(f"  max row error {e:.2e}", flush=True)
    assert e <= (1e-3 if f16 else 1e-5)


def test_w4a8_invalid_scales(dev):
    """An activation scale outside the valid range gives y = bias; a weight group with an invalid
    scale contributes nothing."""
    import torch
    print("\n[w4a8 invalid scales]", flush=True)
    inp, lay = run(dev, 64, 128, 256, 64, 62)
    ws = lay.w_scales_host.copy()
    ws[5, 1] = np.float32(1e-35)
    lay.ws.copy_(torch.from_numpy(ws))
    lay.gemm()
    qa, sa, sw, _ = oracle_ref(inp, 64)
    qw = oracle.quant_w4(inp["w"], 64, sw)
    y = oracle.gemm_w4a8(qa, sa, qw, ws, 64, inp["bias"].astype(np.float64))
    assert oracle.rowwise_error(lay.y.cpu().numpy(), y).max() <= 1e-5
    lay.xs.fill_(float("inf"))
    lay.gemm()
    torch.cuda.synchronize()
    assert np.array_equal(lay.y.cpu().numpy(), np.broadcast_to(inp["bias"], (64, 128)))


@pytest.mark.parametrize("M", [256, 4096])
def test_w4a8_mamba2_in_proj_sampled(dev, M):
    """Mamba2-8B-shaped input projection (K = 4096 -> N = 18560) at M = 256 decode tokens and at
    M = 4096 prefill tokens, one scale per output channel, launched as the benchmark does: sampled
    rows of y against the oracle, all activation codes bit-exact."""
    print(f"\n[w4a8 in_proj M={M}]", flush=True)
    inp, lay = run(dev, M, 18560, 4096, 4096, 63)
    rows = np.array([0, M // 3, M - 1])
    qa, sa, sw, y = oracle_ref(inp, 4096, rows=rows)
    assert np.array_equal(lay.xq.cpu().numpy()[rows], qa)
    e = oracle.rowwise_error(lay.y.cpu().numpy()[rows], y).max()
    print(f"  max row error {e:.2e}", flush=True)
    assert e <= 1e-5
