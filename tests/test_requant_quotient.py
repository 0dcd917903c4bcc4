"""The requantiser forms each v / d from one reciprocal per block and a remainder correction
(csrc/requant.hip).  tests/requant_quotient_check.c restates that arithmetic on the host and
compares it with the IEEE quotient for every e4m3 pair at many scales; this runs it."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_requant_quotient_equals_ieee_division(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not on PATH")
    exe = str(tmp_path / "requant_quotient_check")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           os.path.join(HERE, "requant_quotient_check.c"), "-o", exe, "-lm"])
    r = subprocess.run([exe, "3000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    checks = int(r.stdout.split()[1])
    assert checks > 40_000_000 and "mismatches 0" in r.stdout, r.stdout
