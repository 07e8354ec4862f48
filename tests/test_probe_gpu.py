"""Matrix-core probe on the GPU: the counters it returns are consistent with
the event time, and its products are finite (measurement code, not the path)."""
import numpy as np
import pytest
import torch

import variable_length_flash_jaggedfa_amd as jfa

pytestmark = pytest.mark.gpu


def test_probe_counters_and_rate(gpu):
    wgs, iters = 64, 20000
    sink = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device=gpu)
    clocks = torch.zeros(wgs * 4, dtype=torch.int64, device=gpu)
    jfa.probe_mfma(iters, wgs, sink, clocks)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    jfa.probe_mfma(iters, wgs, sink, clocks)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert torch.isfinite(sink).all() and (sink > 0).all()
    c = clocks.view(wgs, 4).cpu().numpy().astype(np.float64)
    assert (c > 0).all()
    # the constant-rate counter runs at 100 MHz: its span over all loops fits
    # inside the kernel's event time (about 1 ms) and covers most of it
    span_mhz = (c[:, 3].max() - c[:, 2].min()) / (ms * 1e-3) / 1e6
    assert 60.0 < span_mhz < 101.0, span_mhz
    ghz = np.median(c[:, 0] / c[:, 1]) * 0.1
    assert 0.5 < ghz < 3.0, ghz
    # a SIMD's matrix core does at most one 32x32x16 product per 32 core cycles,
    # and each of the workgroup's waves (one per SIMD) issues 4 x iters of them
    assert np.median(c[:, 0]) >= iters * 4 * 32 * 0.99
