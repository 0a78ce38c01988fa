"""The C ABI's host validation built with AddressSanitizer and
UndefinedBehaviorSanitizer (host compiler, no GPU code): kda_api.cpp is linked
against counting stand-ins for the kernel launchers (tests/asan/launch_stubs.cpp)
and driven by tests/asan/validation_driver.cpp, which checks every status code
and that rejected calls reach no launcher, over sizes up to INT_MAX."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_82_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC),
                    reason="needs g++ and the HIP headers")
def test_validation_under_host_sanitizers(tmp_path):
    exe = str(tmp_path / "kda_validation_asan")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", CSRC,
           os.path.join(ROOT, "tests", "asan", "validation_driver.cpp"),
           os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"),
           os.path.join(CSRC, "kda_api.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "all expectations hold" in run.stdout
