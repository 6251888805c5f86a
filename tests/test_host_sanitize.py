"""The C ABI's host-side argument validation under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.cpp is built with g++ (host code only) together with stand-ins for the kernel launchers and
the three HIP runtime calls it makes (tests/host_sanitize/stub_launch.cpp), and driven by a C++
program (tests/host_sanitize/driver.cpp) through every error path and a well-formed call of each
entry point.  No GPU and no HIP runtime are involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "sliding_window_gqa_varlen_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("asan") / "abi_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "abi.cpp"), os.path.join(HERE, "stub_launch.cpp"), os.path.join(HERE, "driver.cpp"),
           "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return out


def test_every_error_path_under_address_and_undefined_behavior_sanitizers(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)  # the driver carries its own sanitizer runtime
    res = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    report = res.stdout + res.stderr
    assert res.returncode == 0, report[-4000:]
    assert "ALL OK" in res.stdout, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
