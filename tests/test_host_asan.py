"""The host library under AddressSanitizer and UBSan (no GPU).

host.cpp (argument checking, slot tables, the chunk budget) is built with
g++ and sanitizers together with stand-ins for the kernel launchers
(tests/asan/launch_stubs.cpp), and tests/asan/host_driver.cpp drives every
entry point with good and bad arguments. A sanitizer report or a failed
check fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_lf_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_library_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    sanitize = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + sanitize +
           [os.path.join(CSRC, "host.cpp"), os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"),
            os.path.join(ROOT, "tests", "asan", "host_driver.cpp"), "-o", exe])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all checks passed" in r.stdout
