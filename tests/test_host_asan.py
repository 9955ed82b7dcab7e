"""The library's host code (plan and partition construction, argument validation, workspace
layouts: csrc/bsa_api.cpp) built for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer
and driven through the C ABI by tests/host_asan/driver.cpp; host_stubs.cpp stands in for the
HIP runtime and the kernel launchers, so no device code runs. Any out-of-bounds access, leak of
a use-after-free or undefined behaviour aborts the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_asan")


def test_host_code_under_address_sanitizer(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "block_sparse_attention_bsa_amd", "csrc", "bsa_api.cpp"),
           os.path.join(HERE, "host_stubs.cpp"), os.path.join(HERE, "driver.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host checks passed" in run.stdout
