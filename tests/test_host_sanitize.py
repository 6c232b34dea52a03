"""Host-side code of libsvdq under AddressSanitizer and UndefinedBehaviorSanitizer.

Only the host translation units are built (g++, no device code) and driven
by tests/native/host_prep_driver.cpp."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_post_quantized_smooth_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_prep_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_prep_asan")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include", "-ffp-contract=off",
           os.path.join(CSRC, "host_prep.cpp"), os.path.join(CSRC, "host_eigen.cpp"),
           os.path.join(ROOT, "tests", "native", "host_prep_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
