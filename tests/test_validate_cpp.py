"""The C ABI's host-side argument checks and workspace layouts (csrc/validate.hpp), compiled
for the CPU with g++ and run under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU:
validate.hpp holds pure host functions).  The checks' own cases live in
tests/cpp/test_validate.cpp."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "cpp", "test_validate.cpp")


def test_validate_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "test_validate")
    # host code only, built by the host compiler; the sanitizer runtimes are linked statically
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-static-libasan", "-static-libubsan",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "linear_selected_token_amd", "csrc"),
           SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    print(r.stdout + r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert ", 0 failed" in r.stdout
