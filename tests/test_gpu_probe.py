"""The instruction-rate probes (measurement support) run on every kind and leave finite or
infinite (the exp chains saturate) values in the sink; bad arguments are refused."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_probe_kinds_run(dev):
    import torch
    import quantized_state_space_amd as qs
    sink = torch.zeros(4 * 256, dtype=torch.float32, device=dev)
    for kind in range(5):
        sink.zero_()
        qs.qssm_probe_rate(kind, 8, 4, sink)
        torch.cuda.synchronize()
        v = sink.cpu().numpy()
        assert not np.isnan(v).all(), kind
    with pytest.raises(qs.QssmError):
        qs.qssm_probe_rate(9, 8, 4, sink)
    with pytest.raises(ValueError):
        qs.qssm_probe_rate(0, 8, 5, sink)
