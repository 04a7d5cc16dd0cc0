"""The GPU encoder replaces IEEE division by a reciprocal and one FMA correction; this
compiles and runs an exhaustive host-side check (all 2^23 divisor mantissas near every
E2M1 rounding threshold) that the E2M1 decisions agree with IEEE division."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_one_correction_quotient_gives_ieee_e2m1_decisions(tmp_path):
    exe = tmp_path / "quotient_check"
    src = os.path.join(HERE, "cpp", "quotient_check.c")
    r = subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", src, "-o", str(exe), "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 E2M1 decisions differ" in r.stdout
