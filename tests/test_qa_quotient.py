"""Host check of the reciprocal-and-residual quotient that the FP8
quantizers (per row, per column, and inside the GEMM) use to quantize bf16 values (page "Operator & Runtime" §5.4.3,
Examples 5-7 and 5-8): over every bf16 pair in its range it must give the
E4M3FN code of the correctly rounded x*448/amax.  The C program is compiled
with gcc here and run on all host cores (about 10 s)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_quotient_rule_codes_exhaustive(tmp_path):
    exe = str(tmp_path / "qa_quotient_check")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                    os.path.join(HERE, "qa_quotient_check.c"), "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600).stdout.split()
    pairs, bad, over = int(out[1]), int(out[3]), int(out[5])
    assert pairs == 983_527_170
    assert bad == 0 and over == 0, out
