"""The measurement-only MFMA / clock probe runs, reports the FLOPs of its
launch, leaves finite per-wave sums and a plausible shader clock."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,wps,rand", [(0, 2, False), (0, 8, True), (1, 1, False), (1, 1, True), (1, 8, False)])
def test_mfma_probe(gpu, kind, wps, rand):
    import measure
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    waves = n_cu * wps * 4
    sink = torch.full((waves,), float("nan"), dtype=torch.float32, device="cuda")
    clocks = torch.zeros((n_cu * wps * 2,), dtype=torch.int64, device="cuda")
    iters = 64
    flop = measure.probe_mfma(kind, wps, iters, rand, sink=sink, clocks=clocks)
    torch.cuda.synchronize()
    per_mfma = 2 * 16 * 16 * 128 if kind == 0 else 2 * 32 * 32 * 16
    assert flop == waves * iters * (8 if kind == 0 else 4) * per_mfma
    assert torch.isfinite(sink).all()
    assert 0.3 < measure.clock_ghz(clocks) < 3.5
    # buffers one element short are rejected before any launch
    with pytest.raises(measure.ProbeError):
        measure.probe_mfma(kind, wps, iters, rand, sink=sink[:-1])
    with pytest.raises(measure.ProbeError):
        measure.probe_mfma(kind, wps, iters, rand, sink=sink, clocks=clocks[:-1])
