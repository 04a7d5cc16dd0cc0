"""The GPU encoders replace IEEE division by a reciprocal and one FMA correction; this
compiles and runs an exhaustive host-side check (all 2^24 divisor mantissas of two binades,
every dividend within six ulps of every decision point) that the rounding decisions agree
with IEEE division: the seven E2M1 thresholds (NVFP4 element codes) and the sixteen
significands of the E4M3 decision points (FP8 KV-cache bytes)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("needs gcc")
    exe = tmp_path_factory.mktemp("qc") / "quotient_check"
    src = os.path.join(HERE, "cpp", "quotient_check.c")
    r = subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", src, "-o", str(exe), "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return str(exe)


@pytest.mark.parametrize("mode", ["e2m1", "e4m3"])
def test_one_correction_quotient_gives_ieee_decisions(checker, mode):
    r = subprocess.run([checker, mode], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert f" 0 {mode.upper()} decisions differ" in r.stdout
