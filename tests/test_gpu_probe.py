"""GPU: the matrix-core rate probe (a measurement utility behind bench.py
--mfma-probe) runs every MFMA form the GEMMs use and reports a finite rate and a
shader clock inside the part's range."""
import math

import pytest
import torch

import block_scaled_fp8_sort_amd as moe
from parity_checks import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", sorted(moe.PROBE_KINDS))
def test_mfma_probe_reports_a_rate(kind):
    say(f"mfma probe kind {kind}: {moe.PROBE_KINDS[kind]}")
    tf, ghz = moe.probe_mfma_rate(kind, iters=2000, device=torch.device("cuda:0"))
    say(f"  {tf:.0f} TFLOP/s at {ghz:.2f} GHz")
    assert math.isfinite(tf) and tf > 0
    assert 0.3 < ghz < 3.0


def test_clock_stamps_bracket_work():
    """Two clock stamps around back-to-back device work: every XCD the stamps
    ran on reports a shader clock inside the part's range (each compute unit
    against its own earlier stamp), the real-time counter advances, and the
    XCD ids are those of an eight-XCD part.  (The
    shader-clock counter follows the actual clock, which drops to its idle
    level when the XCD has no work, so the span holds only queued kernels.)"""
    dev = torch.device("cuda:0")
    say("clock stamps around back-to-back matmuls")
    a = torch.randn(4096, 4096, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):  # the library's set-up and the clock ramp stay outside the span
        torch.mm(a, a, out=b)
    torch.cuda.synchronize()
    s0 = moe.clock_stamp(1024, dev)
    for _ in range(10):
        torch.mm(a, a, out=b)
    s1 = moe.clock_stamp(1024, dev)
    torch.cuda.synchronize()
    h0, h1 = s0.cpu(), s1.cpu()
    assert set((h0[:, 0] // 256).tolist()) <= set(range(8)) and set((h1[:, 0] // 256).tolist()) <= set(range(8))
    assert bool((h1[:, 2].min() > h0[:, 2].max()).item())  # the real-time counter moved on
    clk = moe.shader_clock_ghz(s0, s1)
    say(f"  per-XCD shader clock: {clk}")
    assert len(clk) >= 1
    assert all(0.3 < g < 3.0 for g in clk.values())
