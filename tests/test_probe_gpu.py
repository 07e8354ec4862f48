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


def test_copy_probe_copies(gpu):
    """The HBM copy probe moves every byte (ragged tail, several grid sizes) and
    reports a bandwidth below the 8 TB/s spec."""
    import torch
    import variable_length_flash_jaggedfa_amd as jfa
    n = (37 << 20) + 12  # floats: a size that is no multiple of the grid's stride
    src = torch.arange(n, dtype=torch.float32, device=gpu)
    for wgs in (1, 7, 2048):
        dst = torch.zeros_like(src)
        jfa.probe_copy(src, dst, wgs)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), wgs
    big = torch.ones(256 << 20, dtype=torch.float32, device=gpu)
    out = torch.empty_like(big)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    jfa.probe_copy(big, out, 2048)
    e0.record()
    jfa.probe_copy(big, out, 2048)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * big.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    assert 500 < gbs < 8000, gbs
