"""Host check of the reciprocal-and-residual quotient of the fixed-range
E4M3FN SwiGLU output (page "Operator & Runtime" §5.3.1, Z stored with one
fixed scale factor): for a bf16 range amax in [2^-80, 2^118] and every
product z of two bf16 values with |z| <= amax it must give the E4M3FN code
of the correctly rounded z*448/amax.  The C program is compiled with gcc
here and run on all host cores (a few seconds)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_fixed_range_quotient_codes_exhaustive(tmp_path):
    exe = str(tmp_path / "fixed_quotient_check")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                    os.path.join(HERE, "fixed_quotient_check.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600).stdout.split()
    pairs, bad, over = int(out[1]), int(out[3]), int(out[5])
    assert pairs == 668_369_666
    assert bad == 0 and over == 0, out
