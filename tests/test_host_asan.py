"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU): the front end (csrc/duo_api.cpp) is built
with g++ and the sanitizers against stand-in launchers (tests/asan/) and
driven through layouts, validation, token counts, ragged views and their
workspace offsets, failed launches and the host helpers."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or
                    not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")),
                    reason="needs g++ and the HIP runtime headers")
def test_host_abi_under_address_sanitizer():
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, "host_abi_asan")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "kv_cache_compression_duo_amd", "csrc", "duo_api.cpp"),
           os.path.join(ROOT, "tests", "asan", "stub_launchers.cpp"),
           os.path.join(ROOT, "tests", "asan", "host_abi_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    # the sanitizer runtime is linked in; tolerate other preloaded libraries
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "host ABI checks passed" in r.stdout
