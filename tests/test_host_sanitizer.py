"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU): ptb_api.cpp, the argument checks, the stash and scratch
layouts and the launch arguments, is compiled with g++ against stand-in
launchers that touch every buffer region the API hands to a kernel
(tests/host_sanitizer/stub_launchers.cpp), and driven through every entry
point on host buffers sized by the library's own size queries
(tests/host_sanitizer/abi_driver.cpp).  A planted 4 KB shortfall of the stash
must be reported, which shows that the harness catches what it is for."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "transformer_block_amd", "csrc", "ptb_api.cpp"),
       os.path.join(ROOT, "tests", "host_sanitizer", "stub_launchers.cpp"),
       os.path.join(ROOT, "tests", "host_sanitizer", "abi_driver.cpp")]
ROCM_INCLUDE = "/opt/rocm/include"


def _build(tmp_path, name, extra=()):
    exe = str(tmp_path / name)
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
           *extra, *SRC, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


needs_toolchain = pytest.mark.skipif(
    shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")),
    reason="needs g++ and the ROCm headers")


@needs_toolchain
def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path, "abi_asan")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stderr[-4000:]


@needs_toolchain
def test_the_sanitizer_harness_catches_a_short_stash(tmp_path):
    exe = _build(tmp_path, "abi_asan_planted", ["-DPLANT_SHORT_SAVED"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode != 0
    assert "AddressSanitizer" in res.stderr and "heap-buffer-overflow" in res.stderr
