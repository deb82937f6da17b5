"""The tile scheduler (plan.cpp) and the C ABI's argument validation (capi.cpp),
built for the host alone with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, no device code: the kernel launchers are stubs that abort if reached),
run over random BDLM, varlen and task plans, the document splitter and every
rejection path (tests/sanitize/plan_abi_fuzz.cpp).  Any sanitizer finding
aborts the driver; any plan that disagrees with a brute-force evaluation of the
mask rules fails a check."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "masked_long_context_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"


def test_scheduler_and_abi_under_address_and_ub_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "plan_abi_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}",
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "capi.cpp"), os.path.join(SAN, "launch_stubs.cpp"),
           os.path.join(SAN, "plan_abi_fuzz.cpp"), f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "300"], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert out.strip().splitlines()[-1].startswith("ok:"), out[-2000:]
