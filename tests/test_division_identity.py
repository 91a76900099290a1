"""The fused activation quantization forms fp32(127x)/beta from a reciprocal and two FMAs
(Markstein's correction).  This CPU test checks, exhaustively over every fp32 numerator in
the range that decides an int8 code, that the identity gives the IEEE quotient bit for bit,
for a set of divisors including the hard cases just below powers of two."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_markstein_quotient_matches_ieee_division(tmp_path):
    exe = tmp_path / "markstein_check"
    try:
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-mfma", os.path.join(HERE, "markstein_check.c"),
                               "-o", str(exe), "-lm"])
    except (OSError, subprocess.CalledProcessError) as e:  # pragma: no cover
        pytest.skip(f"no gcc with -mfma: {e}")
    r = subprocess.run([str(exe), "8"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    assert "0 mismatches" in r.stdout
