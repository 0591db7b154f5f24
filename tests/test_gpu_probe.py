"""The measurement aids on the GPU: both probes run through the C-ABI, honour
the timing hook, and report rates between a floor no working GPU of this kind
falls below and the published peaks (which they cannot exceed)."""

import pytest
import torch

from attention_qk_norm_amd import binding as B

pytestmark = pytest.mark.gpu

MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 flop/clk
HBM_PEAK_GBS = 8000.0


def _timed(fn, n=3):
    import bench
    ev = bench.HipEvents()
    best = float("inf")
    for _ in range(n):
        a, b = ev.create(), ev.create()
        B.set_timing_events(a, b)
        fn()
        torch.cuda.synchronize()
        best = min(best, ev.elapsed_ms(a, b))
    return best


def test_mfma_probe_rate():
    dev = torch.device("cuda:0")
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    iters = 4000
    flops = B.mfma_probe_flops(iters)
    assert flops > 0
    ms = _timed(lambda: B.mfma_probe(iters, sink))
    tf = flops / ms / 1e9
    print(f"MFMA probe: {tf:.0f} TFLOP/s")
    assert 500.0 < tf <= MFMA_BF16_PEAK_TFLOPS * 1.01


def test_hbm_read_probe_rate():
    dev = torch.device("cuda:0")
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    src = torch.ones(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    nbytes = B.hbm_read_probe(src, sink)  # warm-up, and the byte count
    assert nbytes == 1 << 30
    ms = _timed(lambda: B.hbm_read_probe(src, sink))
    gbs = nbytes / ms / 1e6
    print(f"HBM read probe: {gbs:.0f} GB/s")
    assert 1000.0 < gbs <= HBM_PEAK_GBS * 1.01
    # a ragged tail (not a multiple of the 8-deep unroll) reads in bounds too
    B.hbm_read_probe(src, sink, nbytes=(1 << 20) + 48)
    torch.cuda.synchronize()
