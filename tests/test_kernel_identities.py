"""Exhaustive CPU checks of the fp32 identities the device quantizer uses in
place of IEEE division (tests/native/kernel_identities.c): the correctly
rounded a / 7 from one multiply and two FMAs, and the correctly rounded 1 / s
of every fp16 group scale from the hardware reciprocal and one Newton step."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_quantizer_division_identities(tmp_path):
    exe = str(tmp_path / "kernel_identities")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off",
                    os.path.join(ROOT, "tests", "native", "kernel_identities.c"), "-o", exe, "-lm"],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
