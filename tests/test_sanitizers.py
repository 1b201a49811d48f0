"""The host planner and the C ABI's validation under the host address and
undefined-behaviour sanitizers (CPU only).

tests/san/fuzz_abi.cpp drives abp_workspace_size, abp_plan_host,
abp_bsr_plan_host and abp_pod_plan_host with a few thousand random batches
(valid ones checked for the Stream-K invariants, broken ones for their error
codes). It is built with g++ from the library's host sources and stub kernel
launchers (tests/san/stubs.cpp): no device code is compiled or run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_bsr_paged_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_planner_and_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "fuzz_abi")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include",
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "api.cpp"),
           os.path.join(ROOT, "tests", "san", "stubs.cpp"),
           os.path.join(ROOT, "tests", "san", "fuzz_abi.cpp"),
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "3000"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "fuzz_abi ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
