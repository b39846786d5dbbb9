"""Every fp32 bit pattern (all 2^32 of them, in chunks) through the GPU's soft-edge encoder and
int8 group quantizer, compared code for code with the oracle's exact encoders (the oracle runs
on the host's cores, chunk by chunk). Covers zeros, denormals, every exponent, infinities and
all NaN payloads."""
import ctypes
import concurrent.futures as cf
import os

import numpy as np
import pytest

import oracle

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CHUNK = 1 << 28
THREADS = min(16, os.cpu_count() or 1)


def oracle_chunk(fn, x, out, extra):
    """Runs an oracle encoder over x (1-D float32) in THREADS slices, each a separate C call."""
    lib = oracle.lib()
    n = x.size
    step = (n + THREADS - 1) // THREADS
    zero = np.zeros(1, np.uint8)
    keep = [zero, *extra]

    def run(k):
        a, b = k * step, min(n, (k + 1) * step)
        if a >= b:
            return
        xs, os_ = x[a:b], out[a:b]
        fn(lib, xs, os_, zero, extra)

    with cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(run, range(THREADS)))
    del keep


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


def softedge_oracle(lib, xs, os_, zero, extra):
    s, L, H, ratio = extra
    lib.orc_softedge_encode(_p(xs), 1, 1, xs.size, None, _p(zero), _p(s), _p(L), _p(H),
                            int(ratio[0]), _p(os_))


def quant_oracle(lib, xs, os_, zero, extra):
    (s,) = extra
    lib.orc_quant_group_x(_p(xs), 1, 1, xs.size, None, _p(zero), _p(s), _p(os_))


@pytest.mark.parametrize("kind", ["softedge", "softedge2", "int8"])
def test_all_fp32_patterns(dev, kind):
    import torch
    import quantized_state_space_amd as qs
    print(f"\n[exhaustive {kind}]", flush=True)
    s = np.float32([0.0371])
    L = np.float32([0.05])
    H = np.float32([2.3])
    g = torch.zeros(1, dtype=torch.uint8, device=dev)
    s_d, L_d, H_d = (torch.from_numpy(v).to(dev) for v in (s, L, H))
    x_d = torch.empty(CHUNK, dtype=torch.float32, device=dev)
    se = kind.startswith("softedge")
    ratio = np.int32([2 if kind == "softedge2" else 4])
    form = qs.QSSM_X_SOFTEDGE2 if kind == "softedge2" else qs.QSSM_X_SOFTEDGE
    c_d = torch.empty(CHUNK, dtype=torch.uint8 if se else torch.int8, device=dev)
    want = np.empty(CHUNK, np.uint8 if se else np.int8)
    for k in range((1 << 32) // CHUNK):
        bits = np.arange(k * CHUNK, (k + 1) * CHUNK, dtype=np.uint32)
        x = bits.view(np.float32)
        x_d.copy_(torch.from_numpy(x))
        if se:
            qs.qssm_softedge_encode(x_d.view(1, 1, CHUNK), g, 1, s_d, L_d, H_d, c_d.view(1, 1, CHUNK),
                                    form=form)
            oracle_chunk(softedge_oracle, x, want, (s, L, H, ratio))
        else:
            qs.qssm_quant_group_x(x_d.view(1, 1, CHUNK), g, 1, s_d, c_d.view(1, 1, CHUNK))
            oracle_chunk(quant_oracle, x, want, (s,))
        got = c_d.cpu().numpy()
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(hex(int(bits[i])), int(got[i]), int(want[i])) for i in bad[:5]]
        print(f"  chunk {k}: {CHUNK} patterns identical", flush=True)
