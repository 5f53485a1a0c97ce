"""The library's host code (api.cpp: argument checks, path choice, workspace
carving) built for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer
and driven through every C-ABI entry point (tests/asan/host_driver.cpp).  The
HIP runtime calls and kernel launchers are stubs; each stub launcher writes
every byte its kernel would write into buffers allocated at exactly the sizes
the library asks for, so a workspace carved too small or a pointer outside the
caller's buffer is a sanitizer report.  CPU only: nothing touches a GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp8_block_scaled_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_asan(tmp_path):
    exe = str(tmp_path / "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "asan", "host_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "host driver ok" in r.stdout
