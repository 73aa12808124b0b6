"""The C ABI layer (api.cpp) and the launch planning (plan.cpp) under gcc's
address and undefined-behaviour sanitizers, on the host alone: the kernel
launchers and the device queries are stubbed (tests/api_host_check.cpp), so
every entry point's validation, dispatch and workspace arithmetic runs and
is checked without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_fp8_linear_amd", "csrc")


def test_api_and_plans_under_sanitizers(tmp_path):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no g++ or no HIP headers")
    exe = str(tmp_path / "api_host_check")
    subprocess.run(["g++", "-std=c++17", "-g", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-isystem", "/opt/rocm/include", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "api_host_check.cpp"),
                    os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-4000:] + r.stderr[-4000:]
