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
