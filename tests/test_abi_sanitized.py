"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

``tests/sanitize/abi_checks.cpp`` drives every host-side check of
``include/mis.h`` (malformed metadata, arguments, labels, workspace sizes,
kernel choices) and the no-device error path; it is compiled with g++
together with ``abi.cpp`` and stand-ins for the GPU launchers
(``tests/sanitize/launch_stubs.cpp``), linked to the HIP host runtime, and
run on the CPU. Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "item_scoring_attention_amd", "csrc")
ROCM = "/opt/rocm"


def test_abi_host_checks_are_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if not gxx or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "abi_checks")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}",
           os.path.join(CSRC, "abi.cpp"), os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "abi_checks.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ)
    # the HIP runtime keeps some allocations until exit; leaks are not what is checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert run.stdout.startswith("ok ")
