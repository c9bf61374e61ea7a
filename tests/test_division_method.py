"""The quantization kernel's reciprocal-corrected quotient gives the IEEE codes.

The kernel forms x / s as fma(e, r, y) with y = x * r, e = fma(-y, s, x) and
r = RN(1 / s) (Markstein's correction).  This test runs that recipe on the
CPU against true binary32 division over every bf16 input for a spread of row
maxima and over random binary32 inputs, including inputs next to the
half-integer multiples of s where a wrong quotient would change the code.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_markstein_quotient_gives_ieee_codes(tmp_path):
    exe = tmp_path / "division_method_check"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           os.path.join(HERE, "division_method_check.c"), "-o", str(exe), "-lm"])
    res = subprocess.run([str(exe), "20000000"], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "mismatches 0" in res.stdout


@pytest.mark.parametrize("divisor", [127, 255, 448])
def test_scale_division_by_constant_is_exact(tmp_path, divisor):
    """Every binary32 row statistic from the 1e-12 guard up gives the IEEE
    scale: / 127 (INT8), / 255 (asymmetric INT8), / 448 (FP8)."""
    exe = tmp_path / "scale_division_check"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           os.path.join(HERE, "scale_division_check.c"), "-o", str(exe), "-lm"])
    res = subprocess.run([str(exe), str(divisor)], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "mismatches 0" in res.stdout and f"divisor {divisor}," in res.stdout
