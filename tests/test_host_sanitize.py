"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer build of the C-ABI argument validation.

api.cpp and attn_plan.cpp (every check the entry points make before any HIP call, the launch
planning and the loss batching) are compiled with g++ for the host together with stand-ins for the
three kernel launchers (tests/sanitize/launch_stubs.cpp) and a driver (tests/sanitize/api_harness.cpp)
that makes valid and invalid calls and checks each status and launch count. No GPU, no HIP calls."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefix_shared_branch_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")


def test_api_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "api_harness")
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "attn_plan.cpp"),
            os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "api_harness.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), *srcs, "-o", exe]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=120)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:]
    assert " 0 failures" in r.stdout
