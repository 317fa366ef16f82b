"""The prefill epilogues form o = acc / l from the row's correctly rounded
reciprocal and one FMA correction per element, and divide only where a
quotient is below 2^-100, zero or NaN.  The declared result is the IEEE
fp32 quotient; this host test checks, on the CPU's IEEE arithmetic, that the
correction gives exactly the quotient's bits over every significand of the
divisor and of the dividend (tests/division_identity.c).  The GPU side of the
same claim is that every GPU test comparing exact quotients (the zero-query
means, the bitwise cases) keeps passing."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_reciprocal_correction_equals_division(tmp_path):
    exe = str(tmp_path / "division_identity")
    r = subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                        os.path.join(HERE, "division_identity.c"), "-o", exe, "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe, "8"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "mismatches 0" in r.stdout, r.stdout
