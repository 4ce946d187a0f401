"""Host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

prsink_host.cpp is compiled host-only with g++ together with stand-ins for the
HIP runtime and the kernel launchers (tests/host_check/hip_stub.cpp) and a
driver (tests/host_check/abi_check.cpp).  The driver runs the dry-run
validation and call-order cases, then streams of blocks on a host buffer that
stands in for the arena (bf16 and fp32, window sizes 1, 2, 3, 5): every region
each kernel launch would touch must lie inside the arena or a caller tensor,
and the logged event records and stream waits must order every consumer after
its producer across two streams (Ref Sink writes of alternating layers, the
clean-KV path and the bank update on a second stream).  No GPU is used.
"""
import os
import shutil
import subprocess

import pytest

from bounded_kv_cache_pr_amd import build

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host_check")


@pytest.fixture(scope="module")
def abi_check(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path_factory.mktemp("san") / "abi_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", build.INCLUDE, "-I", build.CSRC, "-I", HERE,
           os.path.join(build.CSRC, "prsink_host.cpp"), os.path.join(HERE, "hip_stub.cpp"),
           os.path.join(HERE, "abi_check.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, "sanitizer build failed:\n" + res.stderr[-4000:]
    return exe


def test_abi_host_side_under_asan_ubsan(abi_check):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([abi_check], capture_output=True, text=True, timeout=300, env=env)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "abi_check: ALL OK" in res.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out and "LeakSanitizer" not in out
