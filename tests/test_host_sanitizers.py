"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only). qmv_api.cpp (validation, the host codecs, error messages) is
compiled with g++ -fsanitize=address,undefined together with launch stubs
(tests/host_sanitize/launch_stubs.cpp: no GPU code is linked; a launch that
validation lets through returns a stub error) and a driver
(tests/host_sanitize/driver.cpp) that round-trips the codecs on exactly sized
buffers and sends good and bad arguments to the entry points. Any sanitizer
report aborts the driver."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_api_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize_driver")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include", f"-I{ROOT}/include",
           f"-I{ROOT}/bit_matrix_vector_amd/csrc",
           os.path.join(ROOT, "bit_matrix_vector_amd", "csrc", "qmv_api.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "driver.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=300)
    assert b.returncode == 0, b.stdout[-4000:]
    # verify_asan_link_order=0: the environment may preload other libraries
    # ahead of the sanitizer runtime; they are left in place
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=120, env=env)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "HOST-SANITIZE-OK" in r.stdout
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout
