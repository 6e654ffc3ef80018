"""The matrix-core rate probe (include/kvprobe.h) that the benchmark uses
as its measured MFMA denominator: it runs, writes its checksum rows, and
reports the flop count its header states."""
import pytest
import torch

import bit_kv_cache_int2_amd as kv

pytestmark = pytest.mark.gpu


def test_mfma_peak_probe_runs_and_counts():
    blocks, iters = 8, 100
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = kv.mfma_peak_probe(blocks, iters, out)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * iters * 8 * 16384
    assert bool(torch.isfinite(out).all()), "every thread writes a finite checksum"
