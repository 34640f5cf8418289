"""Host checks of floating-point identities the HIP kernels rely on (no GPU)."""

import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_by_15_through_corrected_reciprocal():
    """The quantize kernel forms the group step (hi - lo) / 15 as a product
    with RN(1/15) plus one remainder correction instead of an IEEE division;
    every non-negative finite dividend must give the IEEE quotient."""
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "div15")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "div15_exhaustive.c"),
                        "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "mismatches: 0 of 2139095040" in out.stdout
