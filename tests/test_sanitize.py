"""The library's host code (layout builder, views, upload images, work
lists) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
and run over seeded random layouts and the full-size workloads (CPU only:
tests/sanitize/san_check.cpp links layout.cpp and pack.cpp, which make no
HIP calls)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_factorized_amd", "csrc")
HARNESS = os.path.join(ROOT, "tests", "sanitize", "san_check.cpp")


@pytest.fixture(scope="module")
def san_binary(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("san") / "san_check")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           HARNESS, os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "pack.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def test_host_code_clean_under_asan_ubsan(san_binary):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([san_binary, "200"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "0 failed checks" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
