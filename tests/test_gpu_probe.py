"""The MFMA issue-rate probe (measurement only) runs, reports the FLOPs of
its launch, and leaves finite per-wave sums."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,wps", [(0, 2), (0, 8), (1, 1), (1, 8)])
def test_mfma_probe(kind, wps):
    import sparse_attention_04_amd as dsa
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    waves = n_cu * wps * 4
    sink = torch.full((waves,), float("nan"), dtype=torch.float32, device="cuda")
    iters = 64
    flop = dsa.dsa_probe_mfma(kind, wps, iters, sink=sink)
    torch.cuda.synchronize()
    per_mfma = 2 * 16 * 16 * 128 if kind == 0 else 2 * 32 * 32 * 16
    assert flop == waves * iters * (8 if kind == 0 else 4) * per_mfma
    assert torch.isfinite(sink).all() and (sink > 0).all()
    # a sink one wave short is rejected before any launch
    with pytest.raises(dsa.DSAError):
        dsa.dsa_probe_mfma(kind, wps, iters, sink=sink[:-1])
