"""The activation quantization kernels' division (one IEEE reciprocal per
block, then a product and one fma correction per element) gives the same e4m3
code as the IEEE quotient x / s that the 1x128 rule is written with, for every
scale the rule can produce and every bf16 input of the block (exhaustively),
and for seeded fp32 inputs over every exponent (the SwiGLU output h, which the
gate_up epilogues quantize with the same division).  Checked by a small C
program (tests/quant_div_check.c) on the host."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_division_matches_ieee_quotient(tmp_path):
    exe = str(tmp_path / "quant_div_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", os.path.join(HERE, "quant_div_check.c"), "-lm",
                    "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert r.stdout.count(" 0 mismatches") == 2, r.stdout
