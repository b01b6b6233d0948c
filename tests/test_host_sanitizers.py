"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): ``tests/native/host_abi_checks.cpp`` links the library's host
sources (validation, packing, workspace layouts, chunk and frame loops) with
stand-ins for the device launchers and for the HIP allocation and error
calls, so that allocation and launch failures can be forced."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "volume_rendering_amd", "csrc")


def test_host_abi_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "host_abi_checks")
    srcs = [os.path.join(ROOT, "tests", "native", "host_abi_checks.cpp")] + \
        [os.path.join(CSRC, f) for f in ("abi.cpp", "pack.cpp", "layouts.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", *srcs, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "all" in run.stdout and "checks passed" in run.stdout
    assert "runtime error" not in run.stderr
