"""The host side of the C ABI (pool.cpp, block_manager.cpp) under
AddressSanitizer and UndefinedBehaviorSanitizer: tests/host_sanitize/
host_api_check.cpp drives pool sizing and description, the host validators
and the block manager (forks, copy-on-write appends, refusals, prefix
caching) through fixed cases and a seeded random walk, checking the
invariants pkv.h states after every call.  Built with g++ (host code only)
into a temporary directory and run; any sanitizer report fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_436_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_api_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_api_check")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "host_sanitize", "host_api_check.cpp"),
           os.path.join(CSRC, "pool.cpp"), os.path.join(CSRC, "block_manager.cpp"), "-o", exe]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert b.returncode == 0, b.stdout
    env = dict(os.environ)
    # a library preloaded by the environment may come before the ASan runtime
    env["ASAN_OPTIONS"] = "verify_asan_link_order=0:detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe, "436"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0 and "host api check passed" in r.stdout, r.stdout
    assert "runtime error" not in r.stdout and "ERROR: AddressSanitizer" not in r.stdout, r.stdout
