"""libsvq's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
without a GPU: tests/host/ builds svq_host.cpp and svq_plan.cpp with g++
against stand-ins for the kernel launchers that check every planned launch
(tiles and units inside the matrix, every code load of every wave inside the
packed buffer's code region, LDS within a compute unit, workspace regions
inside the queried workspace)."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "bit_spherical_vector_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path_factory.mktemp("host") / "svq_host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-Wno-deprecated-declarations", "-o", exe,
           os.path.join(CSRC, "svq_host.cpp"), os.path.join(CSRC, "svq_plan.cpp"),
           os.path.join(HOST, "launch_checks.cpp"), os.path.join(HOST, "harness_main.cpp")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


def test_host_code_under_sanitizers(harness):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([harness], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "0 failures" in res.stdout
