"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers are compiled with g++ -fsanitize=address,undefined and run:

* tests/host/api_driver.cpp links the C-ABI layer of libgg
  (moe_expert_grouped_ragged_amd/csrc/gg_api.cpp, the library's host code)
  against a fake HIP runtime (tests/host/fake_hip.cpp: host memory stands in
  for device memory) and recording kernel launchers
  (tests/host/launch_recorder.cpp).  It checks every argument check, the
  launches each entry point makes and their parameters, the
  GG_ERR_UNSUPPORTED_DEVICE path (a device that reports another
  architecture), the GG_DEBUG_VALIDATE offset check and the packing copies.
* tests/host/oracle_driver.cpp calls every function oracle/oracle.cpp
  exports on exact-size buffers with empty experts and rows outside the
  offsets.

A sanitizer report makes the driver exit non-zero, and so does a failed check.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _build_and_run(sources, extra, name):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, name)
        cmd = ["g++", "-std=c++17", *SAN, *extra, *sources, "-o", exe]
        build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert build.returncode == 0, build.stderr[-4000:]
        run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
        assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
        assert "0 of" in run.stdout and "checks failed" in run.stdout, run.stdout
        return run.stdout


def test_api_host_code_under_sanitizers():
    csrc = os.path.join(ROOT, "moe_expert_grouped_ragged_amd", "csrc")
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("HIP headers not installed")
    out = _build_and_run([os.path.join(csrc, "gg_api.cpp"), os.path.join(HOST, "fake_hip.cpp"),
                          os.path.join(HOST, "launch_recorder.cpp"), os.path.join(HOST, "api_driver.cpp")],
                         ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
                          "-I" + csrc, "-I" + HOST], "api_driver")
    print(out)


def test_oracle_under_sanitizers():
    out = _build_and_run([os.path.join(ROOT, "oracle", "oracle.cpp"), os.path.join(HOST, "oracle_driver.cpp")],
                         ["-fopenmp", "-ffp-contract=off"], "oracle_driver")
    print(out)
